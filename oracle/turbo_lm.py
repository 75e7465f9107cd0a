"""CPU oracle for the Lloyd-Max KV-cache formats of the full-attention forward:
the symmetric Turbo4 / Turbo3 / Turbo2 formats (K and V quantised) and the
asymmetric Bf16K + Turbo4V / Turbo3V / Turbo2V formats (K in bf16).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path never does, and this module imports nothing from it.

What the pages fix (``mod.rs``: the ``MetalKvDtype`` variants Turbo4, Turbo3,
Turbo2, Bf16KTurbo4V/3V/2V, ``k_is_rotated`` and the byte table of
``LayerKvCache::alloc``; ``full_attention.rs``: the symmetric and asymmetric
Turbo branches of ``forward_full_attention``):

* a quantised side holds, per element, a b-bit index into a Lloyd-Max
  codebook (b = 4, 3 or 2, so 16, 8 or 4 levels; eight 3-bit indices share 3
  bytes, four 2-bit indices share a byte), plus one E4M3 (FP8) scale for every
  16 elements; the scale is chosen so that the dequantised group has the same
  Euclidean length as the original, and all of it lives in the basis produced
  by the Walsh-Hadamard rotation (mod.rs, ``MetalKvDtype::Turbo4``, ``Turbo3``,
  ``Turbo2``): ``max_seq * kv_dim * b / 8`` data bytes and
  ``max_seq * kv_dim / 16`` scale bytes per side;
* symmetric formats quantise K and V (the query is rotated before attention),
  asymmetric ones keep K in bf16, not rotated (the query is not rotated); V is
  rotated in both, so the attention output is rotated back.

Readings taken where the pages are silent (each also stated at its function):

* V1 the b-bit codebook is the 2^b-level Lloyd-Max (minimum mean-squared
  error) quantiser of the standard normal distribution, which is how the
  rotated coordinates of a group are modelled; it is found by Lloyd's
  iteration in fp64, made exactly symmetric, and used as fp32 levels;
* V2 the indices of a group are chosen on the group normalised by its RMS,
  sigma = sqrt(sum(x^2) / 16) (sum in fp64, rounded to fp32; sigma in fp32):
  index = the number of decision thresholds below x / sigma (fp32), the
  thresholds being the fp32 midpoints of adjacent fp32 levels, i.e. the
  nearest level, ties to the lower one;
* V3 the scale is s = ||x|| / ||c[idx]||, computed in fp64, rounded to fp32,
  then to E4M3 (nearest-even, saturating), so the dequantised group
  ``e4m3(s) * c[idx]`` keeps the group's L2 norm up to that rounding; a zero
  group has scale 0 and indices 0;
* V4 the indices of a head row form a little-endian bit stream, element e at
  bits [b e, b e + b): two per byte (low nibble first) for 4 bits, 8 per 3
  bytes for 3 bits, 4 per byte for 2 bits; data ``[capacity, Hkv, D b / 8]``
  and scales ``[capacity, Hkv, D / 16]`` (one E4M3 byte per group), token-major
  like the bf16 cache;
* V5 the rotation is the orthonormal Walsh-Hadamard transform of a head
  (reading T1 of the Turbo8 oracle); the quantiser's input is the rotated
  vector rounded to fp32;
* V6 the sparse-V gate follows reading T5 of the Turbo8 oracle: softmax over
  every position, value rows whose weight relative to the largest,
  exp(s_t - max s), is below the threshold (1e-3 unless set; 0 disables) are
  left out.

Parity pins live in ``tests/test_oracle_pins.py`` (Lloyd-Max formats section).
"""
from __future__ import annotations

import functools
import math

import numpy as np

from .qwen35 import (act_to_f64, as_qm, bf16_to_f64, f64_to_bf16, mlp_residual, rms_norm,
                     rope_partial, sigmoid)
from .turbo8 import SPARSE_V_DEFAULT, e4m3_decode, e4m3_encode, sparse_v_weights, wht

GROUP = 16

# name -> (quantised K?, bits)
FORMATS = {"turbo4": (True, 4), "turbo3": (True, 3), "turbo2": (True, 2),
           "bf16k_turbo4v": (False, 4), "bf16k_turbo3v": (False, 3), "bf16k_turbo2v": (False, 2)}

# --------------------------------------------------------------------------- codebook


def _normal_cell_mean(a: float, b: float) -> float:
    """E[X | a < X < b] for X ~ N(0, 1) (a may be -inf, b +inf): the density
    difference over the probability, with the probability from erfc on the
    side away from the mean so tail cells keep their precision."""
    pdf = lambda x: 0.0 if math.isinf(x) else math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    if a >= 0:
        prob = 0.5 * (math.erfc(a / math.sqrt(2)) - math.erfc(b / math.sqrt(2)))
    elif b <= 0:
        prob = 0.5 * (math.erfc(-b / math.sqrt(2)) - math.erfc(-a / math.sqrt(2)))
    else:
        prob = 1.0 - 0.5 * math.erfc(-a / math.sqrt(2)) - 0.5 * math.erfc(b / math.sqrt(2))
    return (pdf(a) - pdf(b)) / prob


@functools.lru_cache(maxsize=None)
def _lloyd_max_cached(n: int, iters: int) -> tuple:
    return tuple(_lloyd_max(n, iters).tolist())


def lloyd_max_normal(n: int = 16, iters: int = 20000) -> np.ndarray:
    """Reading V1: the n-level Lloyd-Max quantiser of N(0, 1), float64 (cached)."""
    return np.array(_lloyd_max_cached(n, iters))


def _lloyd_max(n: int, iters: int) -> np.ndarray:
    """Lloyd's iteration: thresholds at the midpoints of adjacent levels, then
    each level moved to the mean of N(0, 1) over its cell, until nothing moves.
    """
    c = np.linspace(-2.5, 2.5, n)
    for _ in range(iters):
        t = (c[:-1] + c[1:]) / 2
        edges = [-math.inf, *t.tolist(), math.inf]
        nc = np.array([_normal_cell_mean(edges[i], edges[i + 1]) for i in range(n)])
        done = np.max(np.abs(nc - c)) < 1e-15
        c = nc
        if done:
            break
    return (c - c[::-1]) / 2  # exactly symmetric


def codebook_f32(bits: int = 4) -> np.ndarray:
    """The levels as the format stores and uses them (fp32)."""
    return lloyd_max_normal(1 << bits).astype(np.float32)


def thresholds_f32(levels: np.ndarray) -> np.ndarray:
    """Reading V2: fp32 midpoints of adjacent fp32 levels."""
    lv = np.asarray(levels, dtype=np.float32)
    return ((lv[:-1] + lv[1:]) * np.float32(0.5)).astype(np.float32)


# --------------------------------------------------------------------------- packing


def pack_indices(idx: np.ndarray, bits: int) -> np.ndarray:
    """Indices [..., n] -> bytes [..., n * bits / 8], little-endian bit stream,
    element e at bits [bits e, bits e + bits) (reading V4)."""
    idx = np.asarray(idx, dtype=np.int64)
    n = idx.shape[-1]
    assert (n * bits) % 8 == 0
    out = np.zeros((*idx.shape[:-1], n * bits // 8), dtype=np.int64)
    for e in range(n):
        for k in range(bits):
            bp = e * bits + k
            out[..., bp // 8] |= ((idx[..., e] >> k) & 1) << (bp % 8)
    return out.astype(np.uint8)


def unpack_indices(packed: np.ndarray, bits: int) -> np.ndarray:
    """Bytes [..., m] -> indices [..., m * 8 / bits] (reading V4)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    n = p.shape[-1] * 8 // bits
    out = np.zeros((*p.shape[:-1], n), dtype=np.int64)
    for e in range(n):
        for k in range(bits):
            bp = e * bits + k
            out[..., e] |= ((p[..., bp // 8] >> (bp % 8)) & 1) << k
    return out


# --------------------------------------------------------------------------- group quantisation


def quantize(x: np.ndarray, bits: int = 4):
    """Rotated values (last axis a multiple of 16) -> (packed indices uint8
    [..., n bits / 8], E4M3 scale codes uint8 [..., n/16]); readings V2-V4."""
    xf = np.asarray(x, dtype=np.float64).astype(np.float32)
    n = xf.shape[-1]
    assert n % GROUP == 0
    g = xf.reshape(*xf.shape[:-1], n // GROUP, GROUP)
    lv = codebook_f32(bits)
    th = thresholds_f32(lv)
    ss = np.sum(g.astype(np.float64) ** 2, axis=-1)                         # exact squares, fp64 sum
    sigma = np.sqrt(ss.astype(np.float32) / np.float32(GROUP)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (g / sigma[..., None]).astype(np.float32)
    idx = np.sum(y[..., None] > th, axis=-1).astype(np.int64)             # thresholds below y
    zero = ss == 0
    idx = np.where(zero[..., None], 0, idx)
    cn = np.sqrt(np.sum(lv.astype(np.float64)[idx] ** 2, axis=-1))
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(zero, 0.0, np.sqrt(ss) / cn)
    sc = e4m3_encode(s.astype(np.float32))
    return pack_indices(idx.reshape(*xf.shape[:-1], n), bits), sc.astype(np.uint8)


def dequantize(packed: np.ndarray, scales_e4m3: np.ndarray, bits: int = 4) -> np.ndarray:
    """Stored indices and scales -> float64 rotated values, e4m3(s) * level."""
    idx = unpack_indices(packed, bits)
    n = idx.shape[-1]
    lv = codebook_f32(bits).astype(np.float64)
    v = lv[idx].reshape(*idx.shape[:-1], n // GROUP, GROUP)
    s = e4m3_decode(scales_e4m3)
    return (v * s[..., None]).reshape(idx.shape)


# 4-bit names kept for the Bf16K + Turbo4V callers
def turbo4_quantize(x):
    return quantize(x, 4)


def turbo4_unpack(packed):
    return unpack_indices(packed, 4)


def turbo4_dequantize(packed, scales):
    return dequantize(packed, scales, 4)


# --------------------------------------------------------------------------- attention and layer


def attention_decode(fmt: str, q: np.ndarray, kv: dict, seq_len: int,
                     sparse_v: float = SPARSE_V_DEFAULT) -> np.ndarray:
    """GQA decode attention over a Lloyd-Max format cache: for a symmetric
    format the query is rotated and scored against the dequantised rotated
    keys, for an asymmetric one the unrotated query against the bf16 keys
    (scale 1/sqrt(D), softmax over [0, seq_len)); the weights, with the rows
    the sparse-V gate skips set to zero (reading V6), apply to the
    dequantised rotated values and the output is rotated back.

    q: [Hq, D] float64; kv: {"k", "v", "v_scales"} (+ "k_scales" when K is
    quantised).  Returns [Hq, D] float64.
    """
    kq, bits = FORMATS[fmt]
    Hq, D = q.shape
    Hkv = kv["k"].shape[1]
    rep = Hq // Hkv
    if kq:
        K = dequantize(kv["k"][:seq_len], kv["k_scales"][:seq_len], bits)
        qq = wht(q)
    else:
        K = bf16_to_f64(kv["k"][:seq_len])
        qq = q
    V = dequantize(kv["v"][:seq_len], kv["v_scales"][:seq_len], bits)
    out = np.empty((Hq, D))
    for h in range(Hq):
        g = h // rep
        s = K[:, g, :] @ qq[h] / math.sqrt(D)
        _, pk = sparse_v_weights(s, sparse_v)
        out[h] = pk @ V[:, g, :]
    return wht(out)


def attention_decode_bf16k_turbo4v(q, kc, vc, vs, seq_len, sparse_v: float = SPARSE_V_DEFAULT):
    return attention_decode("bf16k_turbo4v", q, {"k": kc, "v": vc, "v_scales": vs}, seq_len,
                            sparse_v)


def append(fmt: str, kv: dict, pos: int, k: np.ndarray, v: np.ndarray) -> dict:
    """A copy of the cache with row ``pos`` holding k (bf16, or rotated and
    quantised for a symmetric format) and the rotated, quantised v ([Hkv, D]
    float64, unrotated)."""
    kq, bits = FORMATS[fmt]
    out = {name: np.array(a, copy=True) for name, a in kv.items()}
    if kq:
        out["k"][pos], out["k_scales"][pos] = quantize(wht(k), bits)
    else:
        out["k"][pos] = f64_to_bf16(k)
    out["v"][pos], out["v_scales"][pos] = quantize(wht(v), bits)
    return out


def bf16k_turbo4v_append(kv, pos, k, v):
    return append("bf16k_turbo4v", kv, pos, k, v)


def forward_full_attention(fmt: str, cfg, layer: dict, kv: dict, inv_freq: np.ndarray,
                           x_in: np.ndarray, cache_pos: int, sparse_v: float = SPARSE_V_DEFAULT):
    """One token through one gated full-attention layer with a Lloyd-Max format
    cache (the Turbo branches of ``forward_full_attention``): the bf16 layer's
    steps with the quantising append and the format's attention.
    Returns (x_out float64, new_kv, taps)."""
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
    new_kv = append(fmt, kv, cache_pos, kr, v.reshape(Hkv, D))
    attn = attention_decode(fmt, qr, new_kv, cache_pos + 1, sparse_v)
    ga = attn * sigmoid(gate)
    o = as_qm(layer["o_proj"]) @ ga.reshape(-1)
    r = x + o
    x_out, mt = mlp_residual(cfg, layer, r)
    taps = {"x_norm": xn, "q_full": q_full, "k": k, "v": v, "q_norm_out": qr.reshape(-1),
            "k_norm_out": kr.reshape(-1), "attn_out": attn.reshape(-1),
            "gated_attn": ga.reshape(-1), "o": o, "x_resid": r, "x_out": x_out}
    taps.update(mt)
    return x_out, new_kv, taps


def forward_full_attention_bf16k_turbo4v(cfg, layer, kv, inv_freq, x_in, cache_pos,
                                         sparse_v: float = SPARSE_V_DEFAULT):
    return forward_full_attention("bf16k_turbo4v", cfg, layer, kv, inv_freq, x_in, cache_pos,
                                  sparse_v)
