"""Pins of the oracle's caller-owned stack tail (final norm, lm_head, greedy
token, layer loop) and of the whole-layer forwards of the quantised KV formats.

The stack tail is the part the Module qwen3_5 page leaves to the caller (it
owns the sampler and the weights); the quantised forwards are the Turbo
branches of ``forward_full_attention`` (full_attention.rs page).  Each test
fixes a result by a closed form, a special case, torch's CPU routines or by
composing single-layer calls whose parts are pinned elsewhere; none re-types
an oracle formula to make its expected value.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from oracle import turbo8 as T8
from oracle import turbo_lm as TL


def f32_bits(x):
    return np.float32(x).view(np.uint32).item()


def bf16_bits(x):
    b = f32_bits(x)
    assert b & 0xFFFF == 0, x
    return b >> 16


# --------------------------------------------------------------------------- greedy


def test_greedy_lowest_index_wins_an_exact_tie():
    assert O.greedy(np.array([0.0, 3.0, 1.0, 3.0, 3.0])) == 1
    assert O.greedy(np.array([2.5, 2.5, 2.5])) == 0
    assert O.greedy(np.array([-1.0, -0.5, -0.5, -2.0])) == 1
    # the largest value wins whatever its position, including the last
    assert O.greedy(np.array([1.0, 2.0, 7.0])) == 2
    # ties between values that differ only in the last fp32 bit are not ties
    a = np.float32(1.0)
    b = np.nextafter(a, np.float32(2.0))
    assert O.greedy(np.array([a, b, a], dtype=np.float64)) == 1
    # -0.0 and +0.0 compare equal: the first one wins
    assert O.greedy(np.array([-0.0, 0.0, -1.0])) == 0
    rng = np.random.default_rng(3)
    for _ in range(20):
        v = rng.integers(0, 5, size=64).astype(np.float64)
        top = v.max()
        assert O.greedy(v) == min(i for i in range(64) if v[i] == top)


# --------------------------------------------------------------------------- final norm + lm_head


def _one_hot_rows(vocab, k, cols):
    """Rows n = e_{cols[n]} with scale 1 and bias 0 (code 1 at one column)."""
    codes = np.zeros((vocab, k), np.uint8)
    codes[np.arange(vocab), cols] = 1
    return {"codes": codes, "scales": np.full((vocab, k // 64), bf16_bits(1.0), np.uint16),
            "biases": np.zeros((vocab, k // 64), np.uint16)}


def test_lm_head_one_hot_rows_pick_normed_inputs_closed_form():
    # x = c * 1 has RMS |c|, so the final norm gives w_k * c / sqrt(c^2 + eps); row n of
    # a one-hot lm_head returns that entry for its own column (not the transpose)
    cfg = synth.tiny("f32")
    k, vocab, c = cfg.hidden, 37, 0.75
    cols = (np.arange(vocab) * 7) % k
    w = np.array([bf16_bits(v) for v in (1.0 + (np.arange(k) % 5) / 8.0)], np.uint16)
    x = np.full(k, c, np.float32)
    got = O.lm_head_logits(cfg, w, _one_hot_rows(vocab, k, cols), x)
    wv = 1.0 + (cols % 5) / 8.0
    expect = wv * c / math.sqrt(c * c + cfg.rms_eps)
    assert np.allclose(got, expect, rtol=1e-14, atol=0)


def test_lm_head_group_bias_multiplies_the_group_sum():
    # codes 0, scale 0 and bias b_g on group g: logit = sum_g b_g * sum_{k in g} h_k.
    # With x = c * 1 and unit norm weights every h_k equals c / sqrt(c^2 + eps).
    cfg = synth.tiny("f32")
    k, c = cfg.hidden, -1.5
    G = k // 64
    biases = np.zeros((3, G), np.uint16)
    biases[0, 0] = bf16_bits(0.5)          # row 0: group 0 only
    biases[1, :] = bf16_bits(0.25)         # row 1: every group
    biases[2, G - 1] = bf16_bits(-2.0)     # row 2: the last group only
    lm = {"codes": np.zeros((3, k), np.uint8), "scales": np.zeros((3, G), np.uint16), "biases": biases}
    ones = np.full(k, bf16_bits(1.0), np.uint16)
    got = O.lm_head_logits(cfg, ones, lm, np.full(k, c, np.float32))
    h = c / math.sqrt(c * c + cfg.rms_eps)
    assert np.allclose(got, [0.5 * 64 * h, 0.25 * k * h, -2.0 * 64 * h], rtol=1e-14, atol=0)


def test_lm_head_matches_torch_rms_norm_and_linear(gen):
    cfg = synth.tiny("f32")
    vocab, k = 300, cfg.hidden
    lm = gen.quant("pin.tail.lm", vocab, k)
    fn = gen.norm_weight("pin.tail.fn", k)
    x = gen.act("pin.tail.x", (k,), "f32")
    got = O.lm_head_logits(cfg, fn, lm, x)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    bf = lambda b: t(b.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    W = (bf(lm["scales"]).repeat_interleave(64, dim=1).to(torch.float32)
         * t(lm["codes"]).to(torch.float32)
         + bf(lm["biases"]).repeat_interleave(64, dim=1).to(torch.float32)).to(torch.float64)
    h = torch.nn.functional.rms_norm(t(x).to(torch.float64), (k,), bf(fn), eps=cfg.rms_eps)
    ref = torch.nn.functional.linear(h, W).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert O.greedy(got) == int(torch.argmax(torch.from_numpy(ref)))


# --------------------------------------------------------------------------- the layer loop


def _zero_quant(rows, k):
    return {"codes": np.zeros((rows, k), np.uint8), "scales": np.zeros((rows, k // 64), np.uint16),
            "biases": np.zeros((rows, k // 64), np.uint16)}


def _zeroed(layer):
    out = dict(layer)
    for name, v in layer.items():
        if isinstance(v, dict) and "codes" in v:
            r, k = np.asarray(v["codes"]).shape
            out[name] = _zero_quant(r, k)
    return out


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_stack_of_zero_weight_layers_is_the_identity(gen, act):
    cfg = synth.tiny(act)
    kinds = ["gdn", "full", "gdn", "full"]
    layers = [_zeroed(synth.gdn_layer(gen, cfg, f"pin.zs{i}") if k == "gdn"
                      else synth.full_layer(gen, cfg, f"pin.zs{i}")) for i, k in enumerate(kinds)]
    states = [synth.gdn_state(gen, cfg, f"pin.zs{i}", 0.1, 0.5) if k == "gdn" else None
              for i, k in enumerate(kinds)]
    kvs = [synth.kv_cache(gen, cfg, f"pin.zs{i}", 8, 5) if k == "full" else None
           for i, k in enumerate(kinds)]
    x = gen.act("pin.zs.x", (cfg.hidden,), act)
    x64, x_act, new_states, new_kvs = O.decode_stack_step(cfg, kinds, layers, states, kvs,
                                                          O.rope_inv_freq(1e7, 16), x, 5)
    assert np.array_equal(x64, O.act_to_f64(x, act))
    assert np.array_equal(x_act, x)
    for i, k in enumerate(kinds):
        if k == "full":   # row 5 appended (zero k and v), nothing else touched
            changed = np.nonzero(np.any(new_kvs[i]["k"] != kvs[i]["k"], axis=(1, 2)))[0].tolist()
            assert changed in ([5], [])
            assert np.array_equal(new_kvs[i]["k"][:5], kvs[i]["k"][:5])
            assert np.all(O.bf16_to_f64(new_kvs[i]["v"][5]) == 0)
            assert new_states[i] is None
        else:             # the conv window shifted in a zero input
            assert np.array_equal(new_states[i]["conv1d_state"][:, :3], states[i]["conv1d_state"][:, 1:])
            assert np.all(new_states[i]["conv1d_state"][:, 3] == 0)
            assert new_kvs[i] is None


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_stack_step_is_the_layer_calls_in_order(gen, act):
    # a GDN layer then a full layer equals the two single-layer calls, the residual
    # handed over in the activation dtype, each layer given its own state or cache
    cfg = synth.tiny(act)
    g = synth.gdn_layer(gen, cfg, "pin.pair0")
    f = synth.full_layer(gen, cfg, "pin.pair1")
    st = synth.gdn_state(gen, cfg, "pin.pair0", 0.1, 0.5)
    kv = synth.kv_cache(gen, cfg, "pin.pair1", 8, 3)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    x = gen.act("pin.pair.x", (cfg.hidden,), act)
    x64, x_act, states, kvs = O.decode_stack_step(cfg, ["gdn", "full"], [g, f], [st, None],
                                                  [None, kv], inv, x, 3)
    y1, st1, _ = O.forward_linear_attention(cfg, g, st, x)
    h = O.f64_to_act(y1, act)
    y2, kv2, _ = O.forward_full_attention(cfg, f, kv, inv, h, 3)
    assert np.array_equal(x64, y2)
    assert np.array_equal(x_act, O.f64_to_act(y2, act))
    assert all(np.array_equal(states[0][n], st1[n]) for n in st1)
    assert np.array_equal(kvs[1]["k"], kv2["k"]) and np.array_equal(kvs[1]["v"], kv2["v"])
    # the inputs are left as they were
    assert np.array_equal(kv["k"][3], synth.kv_cache(gen, cfg, "pin.pair1", 8, 3)["k"][3])
    if act == "bf16":   # the hand-over is rounded: the unrounded output differs from it
        assert not np.array_equal(O.act_to_f64(h, act), y1)


# --------------------------------------------------------------------------- quantised-format forwards

_PRE_APPEND_TAPS = ("x_norm", "q_full", "k", "v", "q_norm_out", "k_norm_out")


def _fwd(fmt, cfg, layer, kv, inv, x, pos, **kw):
    if fmt == "turbo8":
        return T8.forward_full_attention_turbo8(cfg, layer, kv, inv, x, pos, **kw)
    return TL.forward_full_attention(fmt, cfg, layer, kv, inv, x, pos, **kw)


def _cache(gen, cfg, fmt, prefix, cap, filled):
    if fmt == "turbo8":
        return synth.kv_cache_turbo8(gen, cfg, prefix, cap, filled)
    return synth.kv_cache_lm(gen, cfg, prefix, cap, filled, fmt)


def _attend(fmt, q, kv, n, sparse_v=0.0):
    if fmt == "turbo8":
        return T8.attention_decode_turbo8(q, kv["k"], kv["k_scales"], kv["v"], kv["v_scales"], n,
                                          sparse_v=sparse_v)
    return TL.attention_decode(fmt, q, kv, n, sparse_v=sparse_v)


FORMATS = ["turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]


@pytest.mark.parametrize("fmt", FORMATS)
def test_quantised_forward_shares_the_bf16_steps_before_the_append(gen, fmt):
    # norm, projections, split, q/k norm and RoPE do not depend on the cache format:
    # every tap up to the append is bit-identical to the bf16 forward's (a query
    # rotated before RoPE, or RoPE at another position, would change q_norm_out)
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, f"pin.q{fmt}")
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    x = gen.act(f"pin.q{fmt}.x", (cfg.hidden,), "f32")
    _, _, tb = O.forward_full_attention(cfg, layer, synth.kv_cache(gen, cfg, "pin.qb", 8, 4),
                                        inv, x, 4)
    _, new_kv, tq = _fwd(fmt, cfg, layer, _cache(gen, cfg, fmt, f"pin.q{fmt}", 8, 4), inv, x, 4,
                         sparse_v=0.0)
    for name in _PRE_APPEND_TAPS:
        assert np.array_equal(tq[name], tb[name]), name
    # the attention consumes the post-RoPE query and the cache as appended
    q = tq["q_norm_out"].reshape(cfg.num_heads, cfg.head_dim)
    assert np.array_equal(tq["attn_out"], _attend(fmt, q, new_kv, 5).reshape(-1))


@pytest.mark.parametrize("fmt", ["turbo8", "turbo3", "bf16k_turbo2v"])
def test_quantised_forward_gate_and_tail(gen, fmt):
    cfg = synth.tiny("f32")
    D = cfg.head_dim
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    x = gen.act(f"pin.t{fmt}.x", (cfg.hidden,), "f32")
    kv = _cache(gen, cfg, fmt, f"pin.t{fmt}", 8, 4)
    # gate rows zero: sigmoid(0) = 1/2 scales the attention output
    layer = synth.full_layer(gen, cfg, f"pin.t{fmt}")
    qp = {n: np.array(a, copy=True) for n, a in layer["q_proj"].items()}
    for h in range(cfg.num_heads):
        rows = slice(2 * h * D + D, 2 * (h + 1) * D)
        for n in qp:
            qp[n][rows] = 0
    gl = dict(layer, q_proj=qp)
    _, _, taps = _fwd(fmt, cfg, gl, kv, inv, x, 4, sparse_v=0.0)
    assert np.array_equal(taps["gated_attn"], 0.5 * taps["attn_out"])
    # o_proj zero: the residual is the input and the MLP tail equals the bf16
    # forward's for the same layer (whose tail does not see the cache either)
    zl = dict(layer, o_proj=_zero_quant(*np.asarray(layer["o_proj"]["codes"]).shape))
    xo, _, tq = _fwd(fmt, cfg, zl, kv, inv, x, 4, sparse_v=0.0)
    xb, _, tb = O.forward_full_attention(cfg, zl, synth.kv_cache(gen, cfg, "pin.tb", 8, 4), inv, x, 4)
    assert np.array_equal(tq["x_resid"], x.astype(np.float64))
    assert np.array_equal(xo, xb)
    for name in ("x_norm2", "gate_act", "up_act"):
        assert np.array_equal(tq[name], tb[name]), name


@pytest.mark.parametrize("fmt", ["turbo4", "turbo3", "turbo2"])
def test_symmetric_append_places_one_row_within_the_quantisation_bound(fmt):
    kq, bits = synth.LM_FORMATS[fmt]
    assert kq
    rng = np.random.default_rng(11 + bits)
    cap, Hkv, D = 6, 2, 64
    nb = D * bits // 8
    kv = {"k": np.zeros((cap, Hkv, nb), np.uint8), "v": np.zeros((cap, Hkv, nb), np.uint8),
          "k_scales": np.zeros((cap, Hkv, D // 16), np.uint8),
          "v_scales": np.zeros((cap, Hkv, D // 16), np.uint8)}
    k, v = rng.standard_normal((Hkv, D)), rng.standard_normal((Hkv, D))
    out = TL.append(fmt, kv, 2, k, v)
    for name in kv:
        changed = np.nonzero(np.any((out[name] != kv[name]).reshape(cap, -1), axis=1))[0].tolist()
        assert changed == [2], name
    # Gaussian Lloyd-Max distortion per coordinate: about 0.117 (2 bits), 0.0345 (3 bits),
    # 0.0095 (4 bits) of the variance; rel error = sqrt of that, plus the E4M3 scale rounding
    bound = {2: 0.40, 3: 0.23, 4: 0.13}[bits]
    for side, ref in (("k", k), ("v", v)):
        back = T8.wht(TL.dequantize(out[side][2], out[side + "_scales"][2], bits))
        assert np.linalg.norm(back - ref) / np.linalg.norm(ref) < bound, side
    # rows beyond the append stay zero: a second append elsewhere leaves row 2 alone
    out2 = TL.append(fmt, out, 4, v, k)
    for name in kv:
        assert np.array_equal(out2[name][2], out[name][2])


# --------------------------------------------------------------------------- sparse-V gate


def _lm_cache(rng, fmt, L, Hkv, D):
    kq, bits = synth.LM_FORMATS[fmt]
    nb = D * bits // 8
    kv = {"v": rng.integers(0, 256, (L, Hkv, nb), dtype=np.uint8),
          "v_scales": T8.e4m3_encode(rng.uniform(0.05, 2.0, (L, Hkv, D // 16)).astype(np.float32))}
    if kq:
        kv["k"] = rng.integers(0, 256, (L, Hkv, nb), dtype=np.uint8)
        kv["k_scales"] = T8.e4m3_encode(rng.uniform(0.05, 2.0, (L, Hkv, D // 16)).astype(np.float32))
        K = T8.wht(TL.dequantize(kv["k"], kv["k_scales"], bits))
    else:
        kv["k"] = O.f64_to_bf16(rng.standard_normal((L, Hkv, D)))
        K = O.bf16_to_f64(kv["k"])
    V = T8.wht(TL.dequantize(kv["v"], kv["v_scales"], bits))
    return kv, K, V


@pytest.mark.parametrize("fmt", ["turbo4", "bf16k_turbo2v"])
@pytest.mark.parametrize("tau", [1e-3, 0.05, 0.3])
def test_sparse_v_keeps_the_softmax_and_drops_only_small_rows(fmt, tau):
    # reference from torch: softmax over all rows, then the value rows whose weight
    # relative to the largest is below tau left out of the weighted sum
    rng = np.random.default_rng(int(tau * 1e4) + len(fmt))
    Hq, Hkv, D, L = 4, 2, 64, 41
    kv, K, V = _lm_cache(rng, fmt, L, Hkv, D)
    q = rng.standard_normal((Hq, D)) * 3
    got = TL.attention_decode(fmt, q, kv, L, sparse_v=tau)
    exact = TL.attention_decode(fmt, q, kv, L, sparse_v=0.0)
    rep = Hq // Hkv
    dropped = 0
    for h in range(Hq):
        Kh = torch.from_numpy(K[:, h // rep, :])
        Vh = torch.from_numpy(V[:, h // rep, :])
        s = Kh @ torch.from_numpy(q[h]) / math.sqrt(D)
        p = torch.softmax(s, dim=0)
        rel = p / p.max()
        assert not torch.any(torch.abs(rel - tau) < 1e-9 * tau)   # no row on the boundary
        keep = rel >= tau
        dropped += int((~keep).sum())
        ref = (p * keep) @ Vh
        assert np.allclose(got[h], ref.numpy(), rtol=1e-10, atol=1e-12)
        # the gated output is within the dropped mass of the exact one
        bound = ((p * ~keep)[:, None] * Vh.abs()).sum(0).numpy()
        assert np.all(np.abs(got[h] - exact[h]) <= bound + 1e-12)
    if tau >= 0.05:
        assert dropped > 0


def test_sparse_v_with_one_dominant_key_closed_form():
    # bf16 keys: row 0 is 8 q / |q|^2 * sqrt(D) so its score is 8, the others are
    # zero (score 0).  Relative weights are then 1 and e^-8 = 3.4e-4: at tau 1e-3 only
    # row 0's value is kept, weighted by 1 / (1 + (L - 1) e^-8).
    fmt, D, L = "bf16k_turbo4v", 64, 9
    q = np.zeros((2, D))
    q[:, 0] = 1.0
    k = np.zeros((L, 1, D))
    k[0, 0, 0] = 8.0 * math.sqrt(D)
    kv = {"k": O.f64_to_bf16(k)}
    rng = np.random.default_rng(4)
    kv["v"] = rng.integers(0, 256, (L, 1, D // 2), dtype=np.uint8)
    kv["v_scales"] = T8.e4m3_encode(rng.uniform(0.05, 2.0, (L, 1, D // 16)).astype(np.float32))
    assert np.all(O.bf16_to_f64(kv["k"]) == k)
    got = TL.attention_decode(fmt, q, kv, L, sparse_v=1e-3)
    v0 = T8.wht(TL.dequantize(kv["v"][0], kv["v_scales"][0], 4))[0]
    p0 = 1.0 / (1.0 + (L - 1) * math.exp(-8.0))
    for h in range(2):
        assert np.allclose(got[h], p0 * v0, rtol=1e-12, atol=1e-14)
    # tau 0 keeps every row: the exact softmax average
    full = TL.attention_decode(fmt, q, kv, L, sparse_v=0.0)
    V = T8.wht(TL.dequantize(kv["v"], kv["v_scales"], 4))[:, 0, :]
    w = np.array([1.0] + [math.exp(-8.0)] * (L - 1))
    assert np.allclose(full[0], (w / w.sum()) @ V, rtol=1e-12, atol=1e-14)


def test_turbo8_sparse_v_matches_the_same_rule():
    rng = np.random.default_rng(21)
    Hq, Hkv, D, L = 4, 1, 64, 30
    kc = rng.integers(0, 0x7F, (L, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 0x7F, (L, Hkv, D), dtype=np.uint8)
    ks = O.f64_to_bf16(rng.uniform(1e-2, 4e-2, (L, Hkv, D // 16)))
    vs = O.f64_to_bf16(rng.uniform(1e-3, 4e-3, (L, Hkv, D // 16)))
    q = rng.standard_normal((Hq, D)) * 2
    tau = 0.1
    got = T8.attention_decode_turbo8(q, kc, ks, vc, vs, L, sparse_v=tau)
    K = torch.from_numpy(T8.turbo8_dequantize(kc, ks)[:, 0, :])      # rotated basis
    V = torch.from_numpy(T8.turbo8_dequantize(vc, vs)[:, 0, :])
    kept = 0
    for h in range(Hq):
        s = K @ torch.from_numpy(T8.wht(q[h])) / math.sqrt(D)
        p = torch.softmax(s, dim=0)
        keep = (p / p.max()) >= tau
        kept += int(keep.sum())
        ref = T8.wht(((p * keep) @ V).numpy())
        assert np.allclose(got[h], ref, rtol=1e-10, atol=1e-12)
    assert 0 < kept < Hq * L


def test_fp32_quant_matrix_is_within_fp32_rounding_of_brute_force(gen):
    # the fp32 evaluation of the stack-sized GEMVs: the dense weights are the same
    # exact fp32 values, the product carries fp32 accumulation error only
    w = gen.quant("pin.qm32", 96, 2560)
    x = gen.act("pin.qm32.x", (2560,), "f32").astype(np.float64)
    q32 = O.QuantMatrix(w, np.float32)
    assert q32.dense().dtype == np.float32
    assert np.array_equal(q32.dense(), O.dequant(w))
    ref = np.array([sum(float(a) * float(b) for a, b in zip(row, x)) for row in O.dequant(w)])
    got = q32 @ x
    assert got.dtype == np.float64
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-5
