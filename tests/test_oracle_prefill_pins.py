"""Pins of the prefill oracle (a token loop over the decode step).

The decode step itself is pinned in ``test_oracle_pins.py``.  What these tests
fix is the part the loop adds: the state carried from token to token, the
cache position and RoPE position of each token, and the causal extent of each
token's attention.  Expected values come from other formulations: the chunked
(WY) form of the gated delta rule solved with a library solver, torch's
depthwise conv1d over the whole sequence, torch's SDPA with a causal mask, and
the closed form of the RoPE angle.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth


def _gdn_case(gen, T, act="f32"):
    cfg = synth.tiny(act)
    layer = synth.gdn_layer(gen, cfg, "pf.gdn")
    st = synth.gdn_state(gen, cfg, "pf.gdn", 0.2, 0.5)
    x = gen.act("pf.gdn.x", (T, cfg.hidden), act)
    return cfg, layer, st, x


def _delta_rule_chunked(S0, q, k, v, g, beta, C):
    """The gated delta rule over a sequence in its chunked form.

    Within a chunk, with L_r the running sum of log g and Delta the rows of
    state corrections, the recurrence S_r = g_r S_{r-1} + k_r delta_r^T,
    delta_r = beta_r (v_r - g_r S_{r-1}^T k_r) unrolls to the unit lower
    triangular system (I + A) Delta = beta v - beta e^L (K S0) with
    A[r, s] = beta_r e^(L_r - L_s) k_r.k_s (s < r); then
    y_r = e^(L_r) S0^T q_r + sum_{s<=r} e^(L_r - L_s) (q_r.k_s) delta_s and
    S_C = e^(L_C) S0 + K^T (e^(L_C - L_s) Delta).
    """
    S = S0.astype(np.float64)
    T = q.shape[0]
    ys = np.empty((T, S.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V = q[sl], k[sl], v[sl]
        L = np.cumsum(np.log(g[sl]))
        b = beta[sl]
        n = len(L)
        decay = np.exp(L[:, None] - L[None, :])
        lower = np.tril(np.ones((n, n)), -1)
        A = b[:, None] * decay * (K @ K.T) * lower
        rhs = b[:, None] * V - (b * np.exp(L))[:, None] * (K @ S)
        D = np.linalg.solve(np.eye(n) + A, rhs)
        P = decay * (Q @ K.T) * np.tril(np.ones((n, n)))
        ys[sl] = np.exp(L)[:, None] * (Q @ S) + P @ D
        S = np.exp(L[-1]) * S + K.T @ (np.exp(L[-1] - L)[:, None] * D)
    return ys, S


@pytest.mark.parametrize("chunk", [4, 16])
def test_prefill_gdn_matches_the_chunked_delta_rule(gen, chunk):
    cfg, layer, st, x = _gdn_case(gen, 37)
    _, new, tp = O.prefill.prefill_linear_attention(
        cfg, layer, st, x, taps=("gdn_qkv_smooth", "gate", "beta", "gdn_y"))
    Hk, Hv, dk, dv = cfg.num_k_heads_lin, cfg.num_v_heads_lin, cfg.k_head_dim_lin, cfg.v_head_dim_lin
    s = tp["gdn_qkv_smooth"]
    q = s[:, :Hk * dk].reshape(-1, Hk, dk)
    k = s[:, Hk * dk:2 * Hk * dk].reshape(-1, Hk, dk)
    v = s[:, 2 * Hk * dk:].reshape(-1, Hv, dv)
    y = tp["gdn_y"].reshape(-1, Hv, dv)
    for j in range(Hv):
        i = j * Hk // Hv
        yj, Sj = _delta_rule_chunked(st["gdn_state"][j], q[:, i], k[:, i], v[:, j],
                                     tp["gate"][:, j].astype(np.float64),
                                     tp["beta"][:, j].astype(np.float64), chunk)
        np.testing.assert_allclose(y[:, j], yj / math.sqrt(dk), rtol=2e-5, atol=2e-6)
        np.testing.assert_allclose(new["gdn_state"][j], Sj, rtol=2e-5, atol=2e-6)


def test_prefill_conv_is_a_depthwise_causal_conv_over_the_sequence(gen):
    cfg, layer, st, x = _gdn_case(gen, 23)
    _, new, tp = O.prefill.prefill_linear_attention(cfg, layer, st, x,
                                                    taps=("gdn_qkv_pre", "gdn_qkv_smooth"))
    raw = tp["gdn_qkv_pre"]                                   # [T, C] conv inputs
    # the window holds earlier inputs as the fp32 state stores them; the newest tap
    # is the token's own unrounded input
    seq = np.concatenate([st["conv1d_state"], raw.T.astype(np.float32)], axis=1)
    seq = seq.astype(np.float64)                              # [C, 4 + T]
    w = O.bf16_to_f64(layer["conv1d_weight"])                 # [C, 4]
    out = torch.nn.functional.conv1d(torch.from_numpy(seq[None, :, 1:]),
                                     torch.from_numpy(w[:, None, :]), groups=w.shape[0])[0]
    out += torch.from_numpy(w[:, 3:] * (raw.T - seq[:, 4:]))
    s = torch.nn.functional.silu(out).numpy().T               # [T, C]
    qk = 2 * cfg.num_k_heads_lin * cfg.k_head_dim_lin
    heads = s[:, :qk].reshape(s.shape[0], -1, cfg.k_head_dim_lin)
    heads = heads / np.sqrt((heads ** 2).sum(-1, keepdims=True) + 1e-6)
    s[:, :qk] = heads.reshape(s.shape[0], -1)
    np.testing.assert_allclose(tp["gdn_qkv_smooth"], s, rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(new["conv1d_state"], seq[:, -4:].astype(np.float32))


def _full_case(gen, T, cache_pos, cap):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "pf.full")
    kv = synth.kv_cache(gen, cfg, "pf.full", cap, cache_pos)
    x = gen.act("pf.full.x", (T, cfg.hidden), "f32")
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    return cfg, layer, kv, x, inv


def test_prefill_attention_is_causal_softmax_over_the_cache(gen):
    T, pos = 11, 5
    cfg, layer, kv, x, inv = _full_case(gen, T, pos, 24)
    _, new, tp = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos,
                                                  taps=("q_norm_out", "attn_out"))
    Hq, Hkv, D = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    L = pos + T
    K = torch.from_numpy(O.bf16_to_f64(new["k"][:L])).permute(1, 0, 2)   # [Hkv, L, D]
    V = torch.from_numpy(O.bf16_to_f64(new["v"][:L])).permute(1, 0, 2)
    K = K.repeat_interleave(Hq // Hkv, 0)
    V = V.repeat_interleave(Hq // Hkv, 0)
    q = torch.from_numpy(tp["q_norm_out"].reshape(T, Hq, D)).permute(1, 0, 2)  # [Hq, T, D]
    mask = torch.arange(L)[None, :] <= (pos + torch.arange(T))[:, None]      # [T, L]
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask)
    np.testing.assert_allclose(tp["attn_out"].reshape(T, Hq, D), ref.permute(1, 0, 2).numpy(),
                               rtol=1e-10, atol=1e-12)
    # rows below the old fill are untouched, rows past the new fill still empty
    assert np.array_equal(new["k"][:pos], kv["k"][:pos])
    assert not new["k"][L:].any() and not new["v"][L:].any()


def test_prefill_rope_position_advances_one_per_token(gen):
    T, pos = 9, 3
    cfg, layer, kv, x, inv = _full_case(gen, T, pos, 16)
    x = np.repeat(x[:1], T, axis=0)                          # the same token T times
    _, _, tp = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, taps=("q_norm_out",))
    D, R = cfg.head_dim, cfg.rotary_dim
    q = tp["q_norm_out"].reshape(T, cfg.num_heads, D)
    z = q[..., :R // 2] + 1j * q[..., R // 2:R]              # rotate-half pairs as complex numbers
    turn = np.angle(z / z[:1])                               # rotation relative to token 0
    want = (np.arange(T)[:, None] * inv.astype(np.float64)[None, :])[:, None, :]
    err = np.angle(np.exp(1j * (turn - want)))
    assert np.abs(err).max() < 1e-5
    np.testing.assert_array_equal(q[..., R:], np.broadcast_to(q[:1, :, R:], q[..., R:].shape))


def test_prefill_in_two_pieces_equals_one_pass(gen):
    cfg, layer, st, x = _gdn_case(gen, 14, "bf16")
    out, new, _ = O.prefill.prefill_linear_attention(cfg, layer, st, x)
    o1, s1, _ = O.prefill.prefill_linear_attention(cfg, layer, st, x[:6])
    o2, s2, _ = O.prefill.prefill_linear_attention(cfg, layer, s1, x[6:])
    assert np.array_equal(out, np.concatenate([o1, o2]))
    for n in ("conv1d_state", "gdn_state"):
        assert np.array_equal(new[n], s2[n])
    T, pos = 10, 2
    cfgf, lay, kv, xf, inv = _full_case(gen, T, pos, 16)
    outf, kvf, _ = O.prefill.prefill_full_attention(cfgf, lay, kv, inv, xf, pos)
    a1, kv1, _ = O.prefill.prefill_full_attention(cfgf, lay, kv, inv, xf[:4], pos)
    a2, kv2, _ = O.prefill.prefill_full_attention(cfgf, lay, kv1, inv, xf[4:], pos + 4)
    assert np.array_equal(outf, np.concatenate([a1, a2]))
    assert np.array_equal(kvf["k"], kv2["k"]) and np.array_equal(kvf["v"], kv2["v"])


# --------------------------------------------------------------------------- quantised caches

QUANT_FORMATS = ["turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]


def _quant_case(gen, fmt, T, cache_pos, cap):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, f"pfq.{fmt}")
    if fmt == "turbo8":
        kv = synth.kv_cache_turbo8(gen, cfg, f"pfq.{fmt}", cap, cache_pos)
    else:
        kv = synth.kv_cache_lm(gen, cfg, f"pfq.{fmt}", cap, cache_pos, fmt)
    x = gen.act(f"pfq.{fmt}.x", (T, cfg.hidden), "f32")
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    return cfg, layer, kv, x, inv


def _turbo_forward(fmt, cfg, layer, kv, inv, x, pos, sparse_v):
    if fmt == "turbo8":
        return O.turbo8.forward_full_attention_turbo8(cfg, layer, kv, inv, x, pos, sparse_v=sparse_v)
    return O.turbo_lm.forward_full_attention(fmt, cfg, layer, kv, inv, x, pos, sparse_v=sparse_v)


@pytest.mark.parametrize("fmt", QUANT_FORMATS)
def test_quantised_prefill_is_the_formats_decode_loop(gen, fmt):
    """A prompt into a quantised cache is the format's decode step per token:
    one token equals the step, the cache rows [pos, pos + T) are the only rows
    written, and two pieces equal one pass (state carried through the cache)."""
    T, pos, cap = 6, 9, 24
    cfg, layer, kv, x, inv = _quant_case(gen, fmt, T, pos, cap)
    for tau in (0.0, 0.05):
        o1, kv1, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x[:1], pos, fmt=fmt, sparse_v=tau)
        r1, rkv1, _ = _turbo_forward(fmt, cfg, layer, kv, inv, x[0], pos, tau)
        assert np.array_equal(o1[0], r1)
        for name in rkv1:
            assert np.array_equal(kv1[name], rkv1[name]), name
    out, new, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt=fmt, sparse_v=0.0)
    for name, a in new.items():
        if not isinstance(a, np.ndarray) or a.ndim == 0 or a.shape[0] != cap:
            continue
        rows = np.nonzero(np.any((a != kv[name]).reshape(cap, -1), axis=1))[0]
        assert set(rows.tolist()) <= set(range(pos, pos + T)), name
        assert np.array_equal(a[:pos], kv[name][:pos]) and np.array_equal(a[pos + T:], kv[name][pos + T:])
    a1, k1, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x[:2], pos, fmt=fmt, sparse_v=0.0)
    a2, k2, _ = O.prefill.prefill_full_attention(cfg, layer, k1, inv, x[2:], pos + 2, fmt=fmt, sparse_v=0.0)
    assert np.array_equal(out, np.concatenate([a1, a2]))
    for name in new:
        assert np.array_equal(np.asarray(new[name]), np.asarray(k2[name])), name


def test_quantised_prefill_honours_the_sparse_v_threshold(gen):
    T, pos, cap = 5, 40, 48
    cfg, layer, kv, x, inv = _quant_case(gen, "turbo4", T, pos, cap)
    o0, _, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt="turbo4", sparse_v=0.0)
    o3, _, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt="turbo4", sparse_v=0.3)
    assert not np.array_equal(o0, o3)
    with pytest.raises(ValueError):
        O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt="turbo5")
