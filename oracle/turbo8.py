"""CPU oracle for the Turbo8 KV-cache format of the full-attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path never does, and this module imports nothing from it.

What the pages fix (``mod.rs``: the ``MetalKvDtype::Turbo8`` variant, the
``LayerKvCache`` struct and its ``alloc`` byte table; ``full_attention.rs``: the
Turbo branch of ``forward_full_attention``):

* K and V are stored in a Walsh-Hadamard-rotated basis, as FP8 E4M3 values
  with one BF16 scale per group of 16 consecutive elements (1.125 bytes per
  element; the data arrays hold ``max_seq * kv_dim`` bytes, the scale arrays
  ``max_seq * kv_dim / 16`` BF16 values);
* the forward rotates the post-RoPE key and the value of each KV head before
  the quantising append, rotates each query head before attention, and applies
  the inverse rotation to the attention output (both sides are rotated).

Readings taken where the pages are silent (each also stated at its function):

* T1 the rotation is the orthonormal Walsh-Hadamard transform of a head
  (``H_D / sqrt(D)``, natural Sylvester order), so its inverse is itself;
* T2 a group's scale is ``bf16(amax / 448)`` (448 is the largest finite E4M3
  value), its codes are E4M3 of ``x / scale`` rounded to nearest-even and
  saturated to +-448; a zero group gets scale 0 and codes 0; the quantiser's
  input is the rotated vector rounded to fp32;
* T3 E4M3 is the OCP "fn" format: bias 7, three mantissa bits, subnormals,
  no infinities, 0x7F and 0xFF are NaN;
* T4 the cache layout follows the bf16 cache: data ``[capacity, Hkv, D]`` and
  scales ``[capacity, Hkv, D / 16]``, token-major;
* T5 the sparse-V gate: the Turbo attention launches take a threshold tau
  (1e-3 unless the caller sets another; 0 turns the gate off) below which a
  position's value row is left out.  The pages give the threshold, not what
  it is compared with.  Reading: with w_t = exp(s_t - max_u s_u), the weight of
  position t relative to the largest one, the softmax is taken over every
  position as usual and only the value rows with w_t < tau are skipped:
  out = sum over {t : w_t >= tau} of p_t V_t, p_t = w_t / sum_u w_u.  A
  streaming kernel that compares against its running maximum instead (never
  above the final one) skips a subset of these rows, so it differs from this
  by at most sum over {t : w_t < tau} of p_t |V_t| per element.

Parity pins live in ``tests/test_oracle_pins.py`` (Turbo8 section).
"""
from __future__ import annotations

import math

import numpy as np

from .qwen35 import (act_to_f64, as_qm, bf16_to_f64, f64_to_bf16, mlp_residual, rms_norm,
                     rope_partial, sigmoid)

E4M3_MAX = 448.0
GROUP = 16
# The sparse-V threshold the Turbo branch uses when the caller does not set one
# (full_attention.rs page, Turbo branch of forward_full_attention); 0 disables it.
SPARSE_V_DEFAULT = 1e-3

# --------------------------------------------------------------------------- rotation


def wht(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform along the last axis (reading T1).

    Butterfly recursion over blocks of doubling width, then the 1/sqrt(D) factor;
    D must be a power of two.  Being orthonormal and symmetric, it is its own
    inverse.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    D = y.shape[-1]
    assert D & (D - 1) == 0, "head_dim must be a power of two"
    h = 1
    while h < D:
        y = y.reshape(*y.shape[:-1], D // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*y.shape[:-3], D)
        h *= 2
    return y / math.sqrt(D)


# --------------------------------------------------------------------------- FP8 E4M3


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (reading T3); NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3 codes, round to nearest-even, saturating (reading T2/T3).

    |x| >= 448 (and infinities) give the largest finite magnitude.  Values below
    the smallest normal 2^-6 are subnormals with a step of 2^-9; a subnormal that
    rounds up to 8 steps is the smallest normal, whose code follows on.
    """
    xf = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(xf).astype(np.int64) << 7
    a = np.abs(xf)
    out = np.zeros(a.shape, dtype=np.int64)
    sat = ~(a < E4M3_MAX)
    sub = a < 2.0 ** -6
    out = np.where(sub, np.rint(np.where(sub, a, 0.0) * 512.0).astype(np.int64), out)
    norm = ~sat & ~sub
    f, E = np.frexp(np.where(norm, a, 1.0))      # a = f * 2^E, f in [0.5, 1)
    e = E - 1                                    # a = (2f) * 2^e, 2f in [1, 2)
    mant = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    out = np.where(norm, ((e + 7) << 3) | mant, out)
    out = np.where(sat, 0x7E, out)
    return (out | sign).astype(np.uint8)


# --------------------------------------------------------------------------- group quantisation


def turbo8_quantize(x: np.ndarray):
    """Rotated values (last axis a multiple of 16) -> (codes uint8, scales bf16 bits).

    Reading T2: the input is taken as fp32; per group of 16 the scale is the
    fp32 quotient amax / 448 rounded to bf16 (nearest-even); codes are E4M3 of
    the fp32 quotient x / scale; a group whose scale is 0 has codes 0.
    """
    xf = np.asarray(x, dtype=np.float64).astype(np.float32)
    n = xf.shape[-1]
    assert n % GROUP == 0
    g = xf.reshape(*xf.shape[:-1], n // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=-1)
    s_bits = f64_to_bf16((amax / np.float32(E4M3_MAX)).astype(np.float32).astype(np.float64))
    s = bf16_to_f64(s_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = g / s[..., None]
    codes = e4m3_encode(y)
    codes = np.where((s == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(xf.shape), s_bits


def turbo8_dequantize(codes: np.ndarray, scales_bf16: np.ndarray) -> np.ndarray:
    """Stored codes and group scales -> float64 rotated values (value * scale, exact)."""
    c = np.asarray(codes)
    n = c.shape[-1]
    v = e4m3_decode(c).reshape(*c.shape[:-1], n // GROUP, GROUP)
    s = bf16_to_f64(scales_bf16)
    return (v * s[..., None]).reshape(c.shape)


# --------------------------------------------------------------------------- attention and layer


def sparse_v_weights(s: np.ndarray, sparse_v: float):
    """Softmax of the scores ``s`` over every position, and the weights with the
    value rows the sparse-V gate skips set to zero (reading T5: a row is skipped
    when ``exp(s_t - max s) < sparse_v``; 0 skips nothing).  Returns (p, p_kept)."""
    w = np.exp(s - s.max())
    p = w / w.sum()
    return p, np.where(w >= sparse_v, p, 0.0)


def attention_decode_turbo8(q: np.ndarray, kc: np.ndarray, ks: np.ndarray, vc: np.ndarray,
                            vs: np.ndarray, seq_len: int,
                            sparse_v: float = SPARSE_V_DEFAULT) -> np.ndarray:
    """GQA decode attention over a Turbo8 cache, in the pages' order: rotate each
    query head, attend with the dequantised rotated keys and values (scale
    1/sqrt(D), softmax over positions [0, seq_len), value rows gated by
    ``sparse_v`` as in reading T5), inverse-rotate the output.

    q: [Hq, D] float64 (unrotated); kc/vc: uint8 [cap, Hkv, D]; ks/vs: bf16
    [cap, Hkv, D/16].  Returns [Hq, D] float64 in the unrotated basis.
    """
    Hq, D = q.shape
    Hkv = kc.shape[1]
    rep = Hq // Hkv
    qr = wht(q)
    K = turbo8_dequantize(kc[:seq_len], ks[:seq_len])
    V = turbo8_dequantize(vc[:seq_len], vs[:seq_len])
    out = np.empty((Hq, D))
    for h in range(Hq):
        g = h // rep
        s = K[:, g, :] @ qr[h] / math.sqrt(D)
        _, pk = sparse_v_weights(s, sparse_v)
        out[h] = pk @ V[:, g, :]
    return wht(out)


def turbo8_append(kv: dict, pos: int, k: np.ndarray, v: np.ndarray) -> dict:
    """Returns a copy of the cache with row ``pos`` holding the rotated, quantised
    key and value ([Hkv, D] float64, unrotated)."""
    out = {name: np.array(a, copy=True) for name, a in kv.items()}
    out["k"][pos], out["k_scales"][pos] = turbo8_quantize(wht(k))
    out["v"][pos], out["v_scales"][pos] = turbo8_quantize(wht(v))
    return out


def forward_full_attention_turbo8(cfg, layer: dict, kv: dict, inv_freq: np.ndarray,
                                  x_in: np.ndarray, cache_pos: int,
                                  sparse_v: float = SPARSE_V_DEFAULT):
    """One token through one gated full-attention layer with a Turbo8 cache (the
    Turbo branch of ``forward_full_attention``): input RMSNorm, q/k/v projections,
    q/gate split, q/k RMSNorm, partial RoPE, rotated quantised append of k and v,
    rotated attention, sigmoid gate, o projection and residual, SwiGLU MLP.

    kv: {"k", "v": uint8 [cap, Hkv, D], "k_scales", "v_scales": bf16 [cap, Hkv, D/16]}.
    Returns (x_out float64, new_kv, taps).
    """
    Hq, Hkv, D, R = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rotary_dim
    x = act_to_f64(x_in, cfg.act_dtype)
    xn = rms_norm(x, layer["input_ln"], cfg.rms_eps)
    q_full = as_qm(layer["q_proj"]) @ xn
    k = as_qm(layer["k_proj"]) @ xn
    v = as_qm(layer["v_proj"]) @ xn
    qh = q_full.reshape(Hq, 2 * D)
    q, gate = qh[:, :D], qh[:, D:]
    qn = rms_norm(q, layer["q_norm"], cfg.rms_eps)
    kn = rms_norm(k.reshape(Hkv, D), layer["k_norm"], cfg.rms_eps)
    qr = rope_partial(qn, cache_pos, inv_freq, R)
    kr = rope_partial(kn, cache_pos, inv_freq, R)
    new_kv = turbo8_append(kv, cache_pos, kr, v.reshape(Hkv, D))
    attn = attention_decode_turbo8(qr, new_kv["k"], new_kv["k_scales"], new_kv["v"],
                                   new_kv["v_scales"], cache_pos + 1, sparse_v)
    ga = attn * sigmoid(gate)
    o = as_qm(layer["o_proj"]) @ ga.reshape(-1)
    r = x + o
    x_out, mt = mlp_residual(cfg, layer, r)
    taps = {"x_norm": xn, "q_full": q_full, "k": k, "v": v, "q_norm_out": qr.reshape(-1),
            "k_norm_out": kr.reshape(-1), "attn_out": attn.reshape(-1),
            "gated_attn": ga.reshape(-1), "o": o, "x_resid": r, "x_out": x_out}
    taps.update(mt)
    return x_out, new_kv, taps
