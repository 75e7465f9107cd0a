"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the decode step by a closed form, a special case
that reduces to a textbook identity, a library routine (torch CPU), or brute
force on tiny inputs.  None of them calls the oracle to make its expected
value, and none re-types the oracle's formula.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(x):
    return np.float32(x).view(np.uint32).item()


def bf16_bits(x):
    """Exact bf16 bit pattern of a value that is representable (truncation of its fp32 bits)."""
    b = f32_bits(x)
    assert b & 0xFFFF == 0, x
    return b >> 16


# --------------------------------------------------------------------------- storage formats

def test_bf16_rounding_ties_and_specials():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert O.f64_to_bf16(np.array([1 + 2 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert O.f64_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82
    # just above the tie rounds up
    assert O.f64_to_bf16(np.array([1 + 2 ** -8 + 2 ** -20]))[0] == 0x3F81
    assert O.f64_to_bf16(np.array([-2.0]))[0] == 0xC000
    assert O.f64_to_bf16(np.array([np.inf]))[0] == 0x7F80
    assert O.f64_to_bf16(np.array([np.nan]))[0] == 0x7FC0
    # round trip of representable values is exact
    vals = np.array([0.0, -0.0, 1.0, 0.75, -3.5, 2.0 ** -100, 65280.0])
    back = O.bf16_to_f64(O.f64_to_bf16(vals))
    assert np.array_equal(back, vals)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(10_000).astype(np.float32)
    ours = O.f64_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------- dequant (O1)

def test_dequant_hand_example():
    # scale 2^-8, bias -1/32, code 200:  200/256 - 1/32 = 0.75 exactly
    w = {"codes": np.full((1, 64), 200, np.uint8),
         "scales": np.array([[bf16_bits(2.0 ** -8)]], np.uint16),
         "biases": np.array([[bf16_bits(-1 / 32)]], np.uint16)}
    d = O.dequant(w)
    assert d.dtype == np.float32
    assert np.all(d == np.float32(0.75))


def test_dequant_group_boundaries():
    # distinct scale/bias per group: column 63 must use group 0, column 64 group 1
    codes = np.arange(256, dtype=np.int64).reshape(1, 256).astype(np.uint8)
    scales = np.array([[bf16_bits(1.0), bf16_bits(2.0), bf16_bits(4.0), bf16_bits(8.0)]], np.uint16)
    biases = np.array([[bf16_bits(0.0), bf16_bits(-1.0), bf16_bits(-2.0), bf16_bits(-3.0)]], np.uint16)
    d = O.dequant({"codes": codes, "scales": scales, "biases": biases})[0]
    for k in range(256):
        g = k // 64
        assert d[k] == (2.0 ** g) * k - g, k


def test_dequant_exact_single_rounding(gen):
    # s*q is exact (<= 16 significant bits) and s*q + b is exact in binary64,
    # so one rounding to fp32 of the exact rational value must give the same bits.
    w = gen.quant("pin.dequant", 8, 128)
    d = O.dequant(w)
    s = w["scales"].astype(np.uint32) << 16
    b = w["biases"].astype(np.uint32) << 16
    for n in range(8):
        for k in range(0, 128, 7):
            sv = Fraction(float(s[n, k // 64:k // 64 + 1].view(np.float32)[0]))
            bv = Fraction(float(b[n, k // 64:k // 64 + 1].view(np.float32)[0]))
            exact = sv * int(w["codes"][n, k]) + bv
            assert d[n, k] == np.float32(float(exact)), (n, k)


def test_synthetic_quantisation_recipe(gen):
    # the generator's codes cover the 8-bit range and the group extremes map near 0 and 255
    w = gen.quant("pin.recipe", 64, 256)
    assert w["codes"].min() == 0 or w["codes"].min() <= 2
    assert w["codes"].max() >= 253
    d = O.dequant(w).astype(np.float64)
    assert abs(d.std() - 0.02) < 0.002


# --------------------------------------------------------------------------- GEMV (O2)

def test_gemv_brute_force(gen):
    w = gen.quant("pin.gemv", 6, 128)
    x = gen.normal_f32("pin.gemv.x", (128,)).astype(np.float64)
    y = O.as_qm(w) @ x
    d = O.dequant(w)
    for n in range(6):
        exact = math.fsum(float(d[n, k]) * float(x[k]) for k in range(128))
        assert abs(y[n] - exact) <= 1e-12 * (1 + abs(exact))


# --------------------------------------------------------------------------- norms

def test_rms_norm_constant_vector_closed_form():
    eps = 1e-6
    w = O.f64_to_bf16(np.linspace(0.5, 1.5, 16))
    wv = O.bf16_to_f64(w)
    for c in (3.0, -0.25, 1e-4):
        out = O.rms_norm(np.full(16, c), w, eps)
        assert np.allclose(out, wv * c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)
    # eps sits under the root: a vector at the scale of sqrt(eps) is shrunk by 1/sqrt(2)
    c = 1e-3
    out = O.rms_norm(np.full(16, c), O.f64_to_bf16(np.ones(16)), 1e-6)
    assert np.allclose(out, 1 / math.sqrt(2), rtol=1e-12)


def test_rms_norm_scale_invariance_and_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32))
    w = O.f64_to_bf16(np.ones(32))
    a = O.rms_norm(x, w, 0.0)
    b = O.rms_norm(1000.0 * x, w, 0.0)
    assert np.allclose(a, b, rtol=1e-13)
    # unit weights and eps 0: every row has mean square exactly 1
    assert np.allclose(np.mean(a * a, axis=-1), 1.0, rtol=1e-13)
    # rows are independent
    assert np.allclose(O.rms_norm(x[2], w, 0.0), a[2])


def test_l2_norm_pythagorean_triple():
    out = O.l2_norm(np.array([[3.0, 4.0]]), 0.0)
    assert np.allclose(out, [[0.6, 0.8]], rtol=1e-15)
    # eps sits under the root of the sum of squares
    out = O.l2_norm(np.array([[3.0, 4.0]]), 1e-6)
    assert np.allclose(out, [[3 / math.sqrt(25 + 1e-6), 4 / math.sqrt(25 + 1e-6)]], rtol=1e-15)


def test_activations_closed_forms():
    assert O.sigmoid(0.0) == 0.5
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1 / (1 + math.exp(-1))) < 1e-15
    assert abs(O.softplus(0.0) - math.log(2)) < 1e-15
    assert O.softplus(50.0) == 50.0
    assert abs(O.softplus(-30.0) - math.exp(-30.0)) < 1e-25
    # library: torch's softplus (threshold 20) and silu in float64
    x = np.linspace(-30, 30, 121)
    assert np.allclose(O.softplus(x), torch.nn.functional.softplus(torch.from_numpy(x)).numpy(),
                       rtol=1e-14, atol=0)
    assert np.allclose(O.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14)


# --------------------------------------------------------------------------- GDN gate / beta

def test_gate_and_beta_invariants():
    a = np.array([-1e3, -5.0, 0.0, 3.0, 8.0])
    dt_bias = O.f64_to_bf16(np.zeros(5))
    a_log = np.array([0.0, 0.5, 1.0, 1.5, 2.0], np.float32)
    g = O.gdn_gate(a, dt_bias, a_log)
    assert g.dtype == np.float32
    assert np.all(g > 0) and np.all(g <= 1)
    assert g[0] == 1.0                         # softplus -> 0 gives no decay
    # a = 0, dt_bias = 0, A_log = 1: exp(-e * ln 2) = 2^-e
    assert abs(float(g[2]) - 2.0 ** (-math.e)) < 1e-7
    # more input means more decay
    a2 = np.linspace(-5, 5, 11)
    g2 = O.gdn_gate(a2, O.f64_to_bf16(np.zeros(11)), np.full(11, 0.7, np.float32))
    assert np.all(np.diff(g2.astype(np.float64)) < 0)
    # dt_bias shifts the input
    g3 = O.gdn_gate(np.array([0.0]), O.f64_to_bf16(np.array([3.0])), np.array([1.0], np.float32))
    g4 = O.gdn_gate(np.array([3.0]), O.f64_to_bf16(np.array([0.0])), np.array([1.0], np.float32))
    assert g3[0] == g4[0]
    b = O.gdn_beta(np.array([0.0, -50.0, 50.0, 1.0]))
    assert b.dtype == np.float32
    assert b[0] == 0.5 and 0 <= b[1] < 1e-20 and b[2] == 1.0
    assert abs(float(b[3]) - 0.7310585786) < 1e-7


# --------------------------------------------------------------------------- conv

def test_conv_zero_state_uses_last_tap():
    C, K = 6, 4
    w = O.f64_to_bf16(np.random.default_rng(5).uniform(-0.5, 0.5, (C, K)))
    x = np.linspace(-1, 1, C)
    st, out = O.conv_update_silu(np.zeros((C, K), np.float32), x, w)
    u = O.bf16_to_f64(w)[:, K - 1] * x
    assert np.allclose(out, u / (1 + np.exp(-u)), rtol=1e-14)
    assert st.dtype == np.float32
    assert np.array_equal(st[:, :K - 1], np.zeros((C, K - 1), np.float32))
    assert np.array_equal(st[:, K - 1], x.astype(np.float32))


def test_conv_matches_torch_depthwise_conv1d():
    rng = np.random.default_rng(6)
    C, K, T = 8, 4, 9
    w = O.f64_to_bf16(rng.uniform(-0.5, 0.5, (C, K)))
    xs = rng.standard_normal((T, C)).astype(np.float32).astype(np.float64)
    st = np.zeros((C, K), np.float32)
    outs = []
    for t in range(T):
        st, o = O.conv_update_silu(st, xs[t], w)
        outs.append(o)
    ref = torch.nn.functional.conv1d(torch.from_numpy(xs.T[None]),
                                     torch.from_numpy(O.bf16_to_f64(w)[:, None, :]),
                                     padding=K - 1, groups=C)[0, :, :T]
    ref = torch.nn.functional.silu(ref).numpy().T
    assert np.allclose(np.array(outs), ref, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- gated delta rule

def _unit(v):
    return v / np.linalg.norm(v)


def test_delta_rule_rank_one_from_zero_state():
    rng = np.random.default_rng(7)
    dk, dv = 8, 6
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    beta = 0.37
    S, y = O.gated_delta_step(np.zeros((dk, dv), np.float32), q, k, v, 1.0, beta)
    assert np.allclose(S, (beta * np.outer(k, v)).astype(np.float32), rtol=1e-6)
    assert np.allclose(y, beta * (q @ k) * v / math.sqrt(dk), rtol=1e-12)


def test_delta_rule_beta_zero_is_pure_decay():
    rng = np.random.default_rng(8)
    dk, dv = 8, 5
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    S, y = O.gated_delta_step(S0, q, k, v, 0.25, 0.0)
    assert np.array_equal(S, (0.25 * S0.astype(np.float64)).astype(np.float32))
    assert np.allclose(y, 0.25 * S0.astype(np.float64).T @ q / math.sqrt(dk), rtol=1e-12)


def test_delta_rule_full_step_overwrites_memory():
    # g = 1, beta = 1, |k| = 1: reading the new state along k returns v exactly
    rng = np.random.default_rng(9)
    dk, dv = 16, 16
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    k = _unit(rng.standard_normal(dk))
    v = rng.standard_normal(dv)
    S, _ = O.gated_delta_step(S0, k, k, v, 1.0, 1.0)
    assert np.allclose(S.astype(np.float64).T @ k, v, rtol=1e-5, atol=1e-5)


def test_delta_rule_unrolled_product_form():
    # S_T = sum_t [prod_{s=T..t+1} g_s (I - b_s k_s k_s^T)] b_t k_t v_t^T + [prod_{s=T..1} ...] S_0
    rng = np.random.default_rng(10)
    dk, dv, T = 6, 4, 4
    S0 = rng.standard_normal((dk, dv))
    ks = [rng.standard_normal(dk) for _ in range(T)]
    vs = [rng.standard_normal(dv) for _ in range(T)]
    gs = [0.9, 0.5, 0.99, 0.7]
    bs = [0.3, 0.8, 0.1, 0.6]

    def A(s):
        return gs[s] * (np.eye(dk) - bs[s] * np.outer(ks[s], ks[s]))

    expect = np.zeros((dk, dv))
    for t in range(T):
        P = np.eye(dk)
        for s in range(T - 1, t, -1):
            P = P @ A(s)
        expect += P @ (bs[t] * np.outer(ks[t], vs[t]))
    P = np.eye(dk)
    for s in range(T - 1, -1, -1):
        P = P @ A(s)
    expect += P @ S0
    # the oracle keeps the state in fp32 between steps; compare at fp32 accuracy
    S = S0.astype(np.float32)
    for t in range(T):
        S, _ = O.gated_delta_step(S, rng.standard_normal(dk), ks[t], vs[t], gs[t], bs[t])
    assert np.allclose(S, expect, rtol=2e-5, atol=2e-5)


# --------------------------------------------------------------------------- RoPE

def test_inv_freq_closed_form():
    getcontext().prec = 40
    f = O.rope_inv_freq(1e7, 64)
    assert f.dtype == np.float32 and f.shape == (32,)
    assert f[0] == 1.0
    # 1e7^(-2/64) = 10^(-7/32)
    exact = Decimal(10) ** (Decimal(-7) / Decimal(32))
    assert f[1] == np.float32(float(exact))
    exact_last = Decimal(10) ** (Decimal(-7 * 62) / Decimal(64))
    assert f[31] == np.float32(float(exact_last))


def test_rope_pass_through_identity_and_norms():
    rng = np.random.default_rng(11)
    H, D, R = 3, 64, 16
    x = rng.standard_normal((H, D))
    inv = O.rope_inv_freq(1e7, R)
    y = O.rope_partial(x, 1234, inv, R)
    assert np.array_equal(y[:, R:], x[:, R:])                 # dims >= R untouched, bit-exact
    assert np.array_equal(O.rope_partial(x, 0, inv, R), x)   # position 0 is the identity
    half = R // 2
    n0 = x[:, :half] ** 2 + x[:, half:R] ** 2
    n1 = y[:, :half] ** 2 + y[:, half:R] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)                   # each pair keeps its length


def test_rope_matches_complex_rotation():
    # rotate-half pairing (i, i+R/2) equals multiplying x_i + j x_{i+R/2} by e^{j theta_i}
    rng = np.random.default_rng(12)
    D, R, pos = 32, 16, 777
    x = rng.standard_normal(D)
    inv = O.rope_inv_freq(1e7, R)
    half = R // 2
    theta = (np.float32(pos) * inv).astype(np.float64)
    z = (x[:half] + 1j * x[half:R]) * np.exp(1j * theta)
    y = O.rope_partial(x, pos, inv, R)
    assert np.allclose(y[:half], z.real, rtol=1e-13, atol=1e-15)
    assert np.allclose(y[half:R], z.imag, rtol=1e-13, atol=1e-15)
    # a unit vector on dim 0 only moves into dim R/2 (not into dim 1)
    e0 = np.zeros(D)
    e0[0] = 1.0
    r = O.rope_partial(e0, 5, inv, R)
    nz = set(np.nonzero(np.abs(r) > 1e-15)[0].tolist())
    assert nz == {0, half}


def test_rope_composition():
    rng = np.random.default_rng(13)
    D, R = 16, 16
    x = rng.standard_normal(D)
    inv = np.array([1.0, 0.5, 0.25, 0.125, 2 ** -4, 2 ** -5, 2 ** -6, 2 ** -7], np.float32)
    # power-of-two frequencies keep the fp32 angles exact, so the rotations compose exactly
    a = O.rope_partial(O.rope_partial(x, 3, inv, R), 5, inv, R)
    b = O.rope_partial(x, 8, inv, R)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- attention

def test_attention_single_position_returns_v():
    rng = np.random.default_rng(14)
    Hq, Hkv, D = 4, 2, 8
    kc = O.f64_to_bf16(rng.standard_normal((3, Hkv, D)))
    vc = O.f64_to_bf16(rng.standard_normal((3, Hkv, D)))
    q = rng.standard_normal((Hq, D)) * 10
    out = O.attention_decode(q, kc, vc, 1)
    V = O.bf16_to_f64(vc)
    for h in range(Hq):
        assert np.array_equal(out[h], V[0, h // 2])


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(15)
    L, Hkv, D = 5, 1, 8
    k = O.f64_to_bf16(np.tile(rng.standard_normal(D), (L, Hkv, 1)))
    vc = O.f64_to_bf16(rng.standard_normal((L, Hkv, D)))
    out = O.attention_decode(rng.standard_normal((2, D)), k, vc, L)
    assert np.allclose(out, O.bf16_to_f64(vc)[:, 0].mean(0), rtol=1e-13)


def test_attention_matches_torch_sdpa_with_gqa():
    rng = np.random.default_rng(16)
    Hq, Hkv, D, L = 8, 2, 16, 37
    kc = O.f64_to_bf16(rng.standard_normal((L + 3, Hkv, D)))
    vc = O.f64_to_bf16(rng.standard_normal((L + 3, Hkv, D)))
    q = rng.standard_normal((Hq, D))
    out = O.attention_decode(q, kc, vc, L)
    K = torch.from_numpy(O.bf16_to_f64(kc)[:L]).permute(1, 0, 2)     # [Hkv, L, D]
    V = torch.from_numpy(O.bf16_to_f64(vc)[:L]).permute(1, 0, 2)
    K = K.repeat_interleave(Hq // Hkv, dim=0)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], K, V)[:, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_attention_ignores_rows_beyond_seq_len():
    rng = np.random.default_rng(17)
    kc = O.f64_to_bf16(rng.standard_normal((6, 1, 4)))
    vc = O.f64_to_bf16(rng.standard_normal((6, 1, 4)))
    q = rng.standard_normal((1, 4))
    a = O.attention_decode(q, kc, vc, 3)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[3:] = 0x7F80
    vc2[3:] = 0x7F80
    assert np.array_equal(a, O.attention_decode(q, kc2, vc2, 3))


# --------------------------------------------------------------------------- layers


def _zero_quant(rows, k):
    return {"codes": np.zeros((rows, k), np.uint8), "scales": np.zeros((rows, k // 64), np.uint16),
            "biases": np.zeros((rows, k // 64), np.uint16)}


def test_gdn_layer_with_zero_weights_is_identity(gen):
    cfg = synth.tiny("f32")
    layer = synth.gdn_layer(gen, cfg, "pin.gdn0")
    for name in ("in_proj_a", "in_proj_b", "in_proj_qkv", "in_proj_z", "out_proj",
                 "gate_proj", "up_proj", "down_proj"):
        r, k = np.asarray(layer[name]["codes"]).shape
        layer[name] = _zero_quant(r, k)
    st = synth.gdn_state(gen, cfg, "pin.gdn0", 0.1, 0.0)
    x = gen.act("pin.gdn0.x", (cfg.hidden,), "f32")
    out, new, _ = O.forward_linear_attention(cfg, layer, st, x)
    assert np.array_equal(out, x.astype(np.float64))
    # conv state (zero here) shifts in a zero column; zero conv inputs give q = k = v = 0
    assert np.array_equal(new["conv1d_state"][:, :3], st["conv1d_state"][:, 1:])
    assert np.all(new["conv1d_state"][:, 3] == 0)
    # zero inputs: gate = exp(-exp(A_log) softplus(dt_bias)), beta = 1/2, k = 0 -> pure decay
    g = O.gdn_gate(np.zeros(cfg.num_v_heads_lin), layer["dt_bias"], layer["a_log"])
    for j in range(cfg.num_v_heads_lin):
        assert np.array_equal(new["gdn_state"][j],
                              (float(g[j]) * st["gdn_state"][j].astype(np.float64)).astype(np.float32))


def test_gdn_layer_head_mapping(gen):
    # v-head j reads k-head j // (Hv/Hk).  Zero the K rows of k-head 0 so only k-head 1
    # has a nonzero key: from a zero state, exactly the v-heads 2 and 3 (of 4) then get
    # a state update; the interleaved mapping j % Hk would update heads 1 and 3 instead.
    cfg = synth.tiny("f32")
    layer = synth.gdn_layer(gen, cfg, "pin.map")
    Hk, dk = cfg.num_k_heads_lin, cfg.k_head_dim_lin
    w = {k: np.array(v, copy=True) for k, v in layer["in_proj_qkv"].items()}
    rows = slice(Hk * dk, Hk * dk + dk)           # K channels of k-head 0
    w["codes"][rows] = 0
    w["scales"][rows] = 0
    w["biases"][rows] = 0
    layer["in_proj_qkv"] = w
    st = synth.gdn_state(gen, cfg, "pin.map")
    x = gen.act("pin.map.x", (cfg.hidden,), "f32")
    _, new, _ = O.forward_linear_attention(cfg, layer, st, x)
    touched = [j for j in range(cfg.num_v_heads_lin) if np.abs(new["gdn_state"][j]).max() > 0]
    assert touched == [2, 3]


def test_full_layer_with_zero_weights_is_identity_and_appends(gen):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "pin.full0")
    for name in ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"):
        r, k = np.asarray(layer[name]["codes"]).shape
        layer[name] = _zero_quant(r, k)
    kv = synth.kv_cache(gen, cfg, "pin.full0", 8, 4)
    sentinel = kv["k"].copy()
    sentinel[4:] = 0x7FC0
    kv = {"k": sentinel.copy(), "v": sentinel.copy()}
    x = gen.act("pin.full0.x", (cfg.hidden,), "f32")
    out, new, _ = O.forward_full_attention(cfg, layer, kv, O.rope_inv_freq(1e7, 16), x, 4)
    assert np.array_equal(out, x.astype(np.float64))
    changed = np.nonzero(np.any(new["k"] != sentinel, axis=(1, 2)))[0].tolist()
    assert changed == [4]
    # zero k, v appended (RoPE may turn a zero into -0, which is still zero)
    assert np.all(O.bf16_to_f64(new["k"][4]) == 0) and np.all(O.bf16_to_f64(new["v"][4]) == 0)


def test_full_layer_sigmoid_gate_half(gen):
    # gate rows zero -> sigmoid(0) = 1/2 scales the attention output
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "pin.gate")
    D = cfg.head_dim
    codes = np.array(layer["q_proj"]["codes"], copy=True)
    sc = np.array(layer["q_proj"]["scales"], copy=True)
    bi = np.array(layer["q_proj"]["biases"], copy=True)
    for h in range(cfg.num_heads):
        rows = slice(2 * h * D + D, 2 * (h + 1) * D)
        codes[rows] = 0
        sc[rows] = 0
        bi[rows] = 0
    layer["q_proj"] = {"codes": codes, "scales": sc, "biases": bi}
    kv = synth.kv_cache(gen, cfg, "pin.gate", 8, 3)
    x = gen.act("pin.gate.x", (cfg.hidden,), "f32")
    _, _, taps = O.forward_full_attention(cfg, layer, kv, O.rope_inv_freq(1e7, 16), x, 3)
    assert np.array_equal(taps["gated_attn"], 0.5 * taps["attn_out"])


def test_preset_matches_pages():
    with open(os.path.join(GOLDEN, "qwen35_4b_preset.json")) as f:
        gold = json.load(f)
    cfg = synth.qwen3_5_4b()
    for k, v in gold.items():
        if k in ("source", "derived"):
            continue
        assert getattr(cfg, k) == v, k
    for k, v in gold["derived"].items():
        if k == "source":
            continue
        assert getattr(cfg, k) == v, k


def test_generator_is_reproducible_and_independent_of_threads(gen):
    a = gen.quant("pin.repro", 4, 128)
    b = synth.Gen(0).quant("pin.repro", 4, 128)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    c = synth.Gen(1).quant("pin.repro", 4, 128)
    assert not np.array_equal(a["codes"], c["codes"])
    # prefix property: a shorter draw is a prefix of a longer one
    x = gen.normal_f32("pin.prefix", (10,))
    y = gen.normal_f32("pin.prefix", (1000,))
    assert np.array_equal(x, y[:10])
    z = gen.normal_f32("pin.stats", (200_000,))
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01


# --------------------------------------------------------------------------- Turbo8 KV cache

from oracle import turbo8 as T8  # noqa: E402


@pytest.mark.parametrize("D", [16, 64, 256])
def test_wht_matches_scipy_hadamard_and_is_an_involution(D):
    import scipy.linalg
    x = np.random.default_rng(D).standard_normal((3, D))
    ref = x @ scipy.linalg.hadamard(D).T / math.sqrt(D)
    assert np.allclose(T8.wht(x), ref, rtol=0, atol=1e-12)
    assert np.allclose(T8.wht(T8.wht(x)), x, rtol=0, atol=1e-12)
    e0 = np.zeros(D)
    e0[0] = 1.0
    assert np.allclose(T8.wht(e0), np.full(D, 1 / math.sqrt(D)), rtol=0, atol=1e-15)


def test_e4m3_decode_matches_torch_float8_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = T8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(7)
    grid = T8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))       # non-negative finite values
    mids = (grid[:-1] + grid[1:]) / 2                                # exact ties (representable in fp32)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.02, 0.02, 2000),
                        mids, -mids, grid, -grid, [0.0, 2.0 ** -10, 3 * 2.0 ** -10]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(T8.e4m3_encode(x), ref)


def test_e4m3_encode_ties_and_saturation_closed_forms():
    enc = T8.e4m3_encode
    assert enc(np.float32(1.0 + 1 / 16)) == 0x38      # tie between 1.0 and 1.125 -> even mantissa
    assert enc(np.float32(1.0 + 3 / 16)) == 0x3A      # tie between 1.125 and 1.25 -> 1.25
    assert enc(np.float32(2.0 ** -10)) == 0x00        # half the smallest subnormal -> 0
    assert enc(np.float32(3 * 2.0 ** -10)) == 0x02    # 1.5 steps -> 2 steps
    assert enc(np.float32(500.0)) == 0x7E and enc(np.float32(-1e30)) == 0xFE
    assert enc(np.float32(np.inf)) == 0x7E


def test_turbo8_group_round_trip_and_error_bound():
    rng = np.random.default_rng(11)
    # a group on the grid: scale a power of two, largest magnitude 448 * scale
    s = 2.0 ** -7
    vals = T8.e4m3_decode(rng.integers(0, 0x7F, 16, dtype=np.uint8)) * s
    vals[3] = 448.0 * s
    codes, sc = T8.turbo8_quantize(vals[None])
    assert O.bf16_to_f64(sc)[0, 0] == s
    assert np.array_equal(T8.turbo8_dequantize(codes, sc)[0], vals)
    # random groups: half an E4M3 step, relative to the value (normals) or to the scale (subnormals)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    codes, sc = T8.turbo8_quantize(x)
    xh = T8.turbo8_dequantize(codes, sc)
    s_el = np.repeat(O.bf16_to_f64(sc), 16, axis=-1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4 * 1.01, s_el * 2.0 ** -10)
    assert np.all(np.abs(xh - x) <= bound)
    # a zero group: scale 0, codes 0
    z = np.zeros((1, 16), np.float32)
    c0, s0 = T8.turbo8_quantize(z)
    assert not c0.any() and not s0.any()


def test_turbo8_attention_equals_sdpa_on_unrotated_dequantised_cache():
    rng = np.random.default_rng(5)
    Hq, Hkv, D, L = 8, 2, 64, 37
    kc = rng.integers(0, 0x7F, (L + 3, Hkv, D), dtype=np.uint8) | (rng.integers(0, 2, (L + 3, Hkv, D), dtype=np.uint8) << 7)
    vc = rng.integers(0, 0x7F, (L + 3, Hkv, D), dtype=np.uint8) | (rng.integers(0, 2, (L + 3, Hkv, D), dtype=np.uint8) << 7)
    ks = O.f64_to_bf16(rng.uniform(1e-3, 4e-3, (L + 3, Hkv, D // 16)))
    vs = O.f64_to_bf16(rng.uniform(1e-3, 4e-3, (L + 3, Hkv, D // 16)))
    q = rng.standard_normal((Hq, D)) * 4
    got = T8.attention_decode_turbo8(q, kc, ks, vc, vs, L, sparse_v=0.0)
    K = torch.from_numpy(T8.wht(T8.turbo8_dequantize(kc[:L], ks[:L]))).permute(1, 0, 2)
    V = torch.from_numpy(T8.wht(T8.turbo8_dequantize(vc[:L], vs[:L]))).permute(1, 0, 2)
    K = K.repeat_interleave(Hq // Hkv, dim=0)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], K, V, scale=1 / math.sqrt(D))[:, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_turbo8_append_places_one_row_within_the_quantisation_bound():
    rng = np.random.default_rng(9)
    cap, Hkv, D = 6, 2, 64
    kv = {"k": np.zeros((cap, Hkv, D), np.uint8), "v": np.zeros((cap, Hkv, D), np.uint8),
          "k_scales": np.zeros((cap, Hkv, D // 16), np.uint16),
          "v_scales": np.zeros((cap, Hkv, D // 16), np.uint16)}
    k, v = rng.standard_normal((Hkv, D)), rng.standard_normal((Hkv, D))
    out = T8.turbo8_append(kv, 4, k, v)
    for name in kv:
        changed = np.nonzero(np.any((out[name] != kv[name]).reshape(cap, -1), axis=1))[0].tolist()
        assert changed == [4], name
    back = T8.wht(T8.turbo8_dequantize(out["k"][4], out["k_scales"][4]))
    assert np.linalg.norm(back - k) / np.linalg.norm(k) < 2.0 ** -4


# --------------------------------------------------------------------------- Turbo4V KV cache (bf16 K)

from oracle import turbo_lm as T4  # noqa: E402


@pytest.mark.parametrize("n", [4, 8, 16])
def test_lloyd_max_codebook_meets_lloyds_conditions_by_quadrature(n):
    from scipy import integrate, stats
    c = T4.lloyd_max_normal(n)
    assert c.shape == (n,) and np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    t = [-np.inf, *((c[:-1] + c[1:]) / 2), np.inf]
    for i in range(n):
        mass = stats.norm.cdf(t[i + 1]) - stats.norm.cdf(t[i]) if t[i] < 0 else \
            stats.norm.sf(t[i]) - stats.norm.sf(t[i + 1])
        first = integrate.quad(lambda x: x * stats.norm.pdf(x), t[i], t[i + 1], epsabs=1e-14)[0]
        assert abs(first / mass - c[i]) < 1e-9, i      # each level is the mean of its cell


@pytest.mark.parametrize("n", [4, 8, 16])
def test_lloyd_max_codebook_agrees_with_kmeans_on_gaussian_samples(n):
    rng = np.random.default_rng(123)
    x = np.sort(rng.standard_normal(1 << 20))
    lv = np.quantile(x, (np.arange(n) + 0.5) / n)
    for _ in range(200):                               # 1-D k-means on the samples
        t = (lv[:-1] + lv[1:]) / 2
        cell = np.searchsorted(t, x)
        lv = np.array([x[cell == i].mean() for i in range(n)])
    assert np.max(np.abs(lv - T4.lloyd_max_normal(n))) < 0.02
    # and the distortion is the smallest among nearby codebooks (a minimum)
    def mse(levels):
        t = (levels[:-1] + levels[1:]) / 2
        return np.mean((x - levels[np.searchsorted(t, x)]) ** 2)
    base = mse(T4.lloyd_max_normal(n))
    for k in range(n // 2):
        bumped = T4.lloyd_max_normal(n).copy()
        bumped[k] += 0.05
        bumped[n - 1 - k] -= 0.05
        assert mse(bumped) > base


def test_packing_is_a_little_endian_bit_stream():
    assert T4.pack_indices(np.arange(8), 3).tolist() == [0x88, 0xC6, 0xFA]
    assert T4.pack_indices(np.array([0, 1, 2, 3]), 2).tolist() == [0xE4]
    assert T4.pack_indices(np.array([1, 14]), 4).tolist() == [0xE1]
    rng = np.random.default_rng(4)
    for bits in (2, 3, 4):
        idx = rng.integers(0, 1 << bits, (3, 5, 32))
        packed = T4.pack_indices(idx, bits)
        assert packed.shape == (3, 5, 32 * bits // 8)
        assert np.array_equal(T4.unpack_indices(packed, bits), idx)


def test_turbo4_packing_low_nibble_first():
    idx = np.arange(16) % 16
    packed = (idx[0::2] | (idx[1::2] << 4)).astype(np.uint8)
    assert np.array_equal(T4.turbo4_unpack(packed), idx)
    assert packed[0] == 0x10 and packed[7] == 0xFE


def test_turbo4_indices_are_nearest_levels_and_the_norm_is_kept():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((200, 64)) * np.exp(rng.uniform(-4, 4, (200, 1)))).astype(np.float32)
    packed, sc = T4.turbo4_quantize(x)
    idx = T4.turbo4_unpack(packed).reshape(200, 4, 16)
    g = x.reshape(200, 4, 16).astype(np.float64)
    lv = T4.codebook_f32().astype(np.float64)
    rms = np.sqrt(np.mean(g ** 2, axis=-1, keepdims=True))
    brute = np.argmin(np.abs((g / rms)[..., None] - lv), axis=-1)
    assert np.mean(brute == idx) > 0.999             # ties and fp32-vs-fp64 edges aside
    assert np.all(np.abs(brute - idx) <= 1)
    # the scale is the norm ratio itself, up to its E4M3 rounding (half a step:
    # 2^-4 relative for normals, 2^-10 absolute below 2^-6), so the norm is kept
    # to that same error
    s = np.linalg.norm(g, axis=-1) / np.linalg.norm(lv[idx], axis=-1)
    err = np.maximum(s * 2.0 ** -4, 2.0 ** -10) * 1.001
    assert np.all(np.abs(T8.e4m3_decode(sc) - s) <= err)
    xh = T4.turbo4_dequantize(packed, sc).reshape(200, 4, 16)
    ratio = np.linalg.norm(xh, axis=-1) / np.linalg.norm(g, axis=-1)
    assert np.all(np.abs(ratio - 1) <= err / s)
    z = np.zeros((1, 16), np.float32)
    p0, s0 = T4.turbo4_quantize(z)
    assert not p0.any() and not s0.any()


@pytest.mark.parametrize("bits", [2, 3])
def test_low_bit_indices_are_nearest_levels_and_the_norm_is_kept(bits):
    rng = np.random.default_rng(22 + bits)
    x = (rng.standard_normal((100, 32)) * np.exp(rng.uniform(-3, 3, (100, 1)))).astype(np.float32)
    packed, sc = T4.quantize(x, bits)
    assert packed.shape == (100, 32 * bits // 8) and sc.shape == (100, 2)
    idx = T4.unpack_indices(packed, bits).reshape(100, 2, 16)
    g = x.reshape(100, 2, 16).astype(np.float64)
    lv = T4.codebook_f32(bits).astype(np.float64)
    rms = np.sqrt(np.mean(g ** 2, axis=-1, keepdims=True))
    brute = np.argmin(np.abs((g / rms)[..., None] - lv), axis=-1)
    assert np.mean(brute == idx) > 0.999 and np.all(np.abs(brute - idx) <= 1)
    s = np.linalg.norm(g, axis=-1) / np.linalg.norm(lv[idx], axis=-1)
    err = np.maximum(s * 2.0 ** -4, 2.0 ** -10) * 1.001
    assert np.all(np.abs(T8.e4m3_decode(sc) - s) <= err)


@pytest.mark.parametrize("fmt", ["turbo4", "turbo3", "turbo2", "bf16k_turbo3v", "bf16k_turbo2v"])
def test_lloyd_max_format_attention_equals_sdpa(fmt):
    kq, bits = T4.FORMATS[fmt]
    rng = np.random.default_rng(31)
    Hq, Hkv, D, L = 8, 2, 64, 23
    nb = D * bits // 8
    kv = {"v": rng.integers(0, 256, (L + 2, Hkv, nb), dtype=np.uint8),
          "v_scales": T8.e4m3_encode(rng.uniform(0.05, 2.0, (L + 2, Hkv, D // 16)).astype(np.float32))}
    if kq:
        kv["k"] = rng.integers(0, 256, (L + 2, Hkv, nb), dtype=np.uint8)
        kv["k_scales"] = T8.e4m3_encode(rng.uniform(0.05, 2.0, (L + 2, Hkv, D // 16)).astype(np.float32))
        K = T8.wht(T4.dequantize(kv["k"][:L], kv["k_scales"][:L], bits))
    else:
        kv["k"] = O.f64_to_bf16(rng.standard_normal((L + 2, Hkv, D)))
        K = O.bf16_to_f64(kv["k"][:L])
    q = rng.standard_normal((Hq, D)) * 3
    got = T4.attention_decode(fmt, q, kv, L, sparse_v=0.0)
    V = T8.wht(T4.dequantize(kv["v"][:L], kv["v_scales"][:L], bits))
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], Kt, Vt, scale=1 / math.sqrt(D))[:, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_turbo4v_attention_equals_sdpa_on_dequantised_values():
    rng = np.random.default_rng(6)
    Hq, Hkv, D, L = 8, 2, 64, 29
    kc = O.f64_to_bf16(rng.standard_normal((L + 2, Hkv, D)))
    vc = rng.integers(0, 256, (L + 2, Hkv, D // 2), dtype=np.uint8)
    vs = T8.e4m3_encode(rng.uniform(0.05, 2.0, (L + 2, Hkv, D // 16)).astype(np.float32))
    q = rng.standard_normal((Hq, D)) * 3
    got = T4.attention_decode_bf16k_turbo4v(q, kc, vc, vs, L, sparse_v=0.0)
    K = torch.from_numpy(O.bf16_to_f64(kc[:L])).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    V = torch.from_numpy(T8.wht(T4.turbo4_dequantize(vc[:L], vs[:L]))).permute(1, 0, 2)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], K, V, scale=1 / math.sqrt(D))[:, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_bf16k_turbo4v_append_places_one_row():
    rng = np.random.default_rng(8)
    cap, Hkv, D = 5, 2, 64
    kv = {"k": np.zeros((cap, Hkv, D), np.uint16), "v": np.zeros((cap, Hkv, D // 2), np.uint8),
          "v_scales": np.zeros((cap, Hkv, D // 16), np.uint8)}
    k, v = rng.standard_normal((Hkv, D)), rng.standard_normal((Hkv, D))
    out = T4.bf16k_turbo4v_append(kv, 3, k, v)
    for name in kv:
        changed = np.nonzero(np.any((out[name] != kv[name]).reshape(cap, -1), axis=1))[0].tolist()
        assert changed == [3], name
    assert np.array_equal(out["k"][3], O.f64_to_bf16(k))
    back = T8.wht(T4.turbo4_dequantize(out["v"][3], out["v_scales"][3]))
    assert np.linalg.norm(back - v) / np.linalg.norm(v) < 0.2   # 4-bit Gaussian codebook: about 0.1


# --------------------------------------------------------------------------- Mode B (diagnostic)


def _bf16_exact(x):
    x = np.asarray(x, dtype=np.float64)
    return np.array_equal(O.bf16_to_f64(O.f64_to_bf16(x)), x)


def test_mode_b_rounds_exactly_the_bf16_buffers(gen):
    """Mode B keeps in bf16 what the pages store in bf16 (GEMV outputs, the smoothed
    qkv, the residual stream) and stays within bf16 rounding of Mode A."""
    cfg = synth.tiny("bf16")
    layer = synth.gdn_layer(gen, cfg, "pin.mb")
    st = synth.gdn_state(gen, cfg, "pin.mb", 0.1, 0.5)
    x = gen.act("pin.mb.x", (cfg.hidden,), "bf16")
    oa, sa, ta = O.forward_linear_attention(cfg, layer, st, x)
    ob, sb, tb = O.forward_linear_attention(cfg, layer, st, x, mode="B")
    for name in ("dt_raw", "b_raw", "gdn_qkv_pre", "z", "gdn_qkv_smooth", "gdn_out", "gdn_x_resid",
                 "gate_act", "up_act"):
        assert _bf16_exact(tb[name]), name
        assert not _bf16_exact(ta[name]), name   # Mode A leaves them unrounded
    assert _bf16_exact(ob)
    assert np.linalg.norm(ob - oa) / np.linalg.norm(oa) < 1e-2
    assert np.linalg.norm(sb["gdn_state"] - sa["gdn_state"]) / np.linalg.norm(sa["gdn_state"]) < 1e-2
    full = synth.full_layer(gen, cfg, "pin.mbf")
    kv = synth.kv_cache(gen, cfg, "pin.mbf", 8, 3)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    fa, _, fta = O.forward_full_attention(cfg, full, kv, inv, x, 3)
    fb, _, ftb = O.forward_full_attention(cfg, full, kv, inv, x, 3, mode="B")
    for name in ("q_full", "k", "v", "o", "x_resid", "gate_act", "up_act"):
        assert _bf16_exact(ftb[name]), name
    assert np.linalg.norm(fb - fa) / np.linalg.norm(fa) < 1e-2
    with pytest.raises(ValueError):
        O.forward_linear_attention(cfg, layer, st, x, mode="C")
