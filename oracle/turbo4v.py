"""CPU oracle for the asymmetric Bf16K + Turbo4V KV-cache format of the
full-attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path never does, and this module imports nothing from it.

What the pages fix (``mod.rs``: the ``MetalKvDtype::Turbo4`` and
``Bf16KTurbo4V`` variants and the byte table of ``LayerKvCache::alloc``;
``full_attention.rs``: the asymmetric branch of ``forward_full_attention``):

* K is stored in bf16 and is not rotated, so the query is not rotated either;
* V is stored as Turbo4: 4-bit indices into a Lloyd-Max codebook and one FP8
  E4M3 scale per group of 16 that keeps the group's L2 norm, in the
  Walsh-Hadamard-rotated basis (V data ``max_seq * kv_dim / 2`` bytes, V scales
  ``max_seq * kv_dim / 16`` bytes: 0.5625 bytes per element);
* V is rotated before the append, so the attention output is rotated back.

Readings taken where the pages are silent (each also stated at its function):

* V1 the codebook is the 16-level Lloyd-Max (minimum mean-squared error)
  quantiser of the standard normal distribution, which is how the rotated
  coordinates of a group are modelled; it is found by Lloyd's iteration in
  fp64 and used as fp32 levels;
* V2 the indices of a group are chosen on the group normalised by its RMS,
  sigma = sqrt(sum(x^2) / 16) (sum in fp64, rounded to fp32; sigma in fp32):
  index = the number of decision thresholds below x / sigma (fp32), the
  thresholds being the fp32 midpoints of adjacent fp32 levels, i.e. the
  nearest level, ties to the lower one;
* V3 the scale is s = ||x|| / ||c[idx]||, computed in fp64, rounded to fp32,
  then to E4M3 (nearest-even, saturating), so the dequantised group
  ``e4m3(s) * c[idx]`` keeps the group's L2 norm up to that rounding; a zero
  group has scale 0 and indices 0;
* V4 two indices per byte, element 2i in the low nibble of byte i; data
  ``[capacity, Hkv, D / 2]`` and scales ``[capacity, Hkv, D / 16]`` (one E4M3
  byte per group), token-major like the bf16 cache;
* V5 the rotation is the orthonormal Walsh-Hadamard transform of a head
  (reading T1 of the Turbo8 oracle); the quantiser's input is the rotated
  vector rounded to fp32;
* V6 attention is exact over all positions (the pages' optional sparse-V gate
  is not applied, as for Turbo8).

Parity pins live in ``tests/test_oracle_pins.py`` (Turbo4V section).
"""
from __future__ import annotations

import functools
import math

import numpy as np

from .qwen35 import (act_to_f64, as_qm, bf16_to_f64, f64_to_bf16, mlp_residual, rms_norm,
                     rope_partial, sigmoid)
from .turbo8 import e4m3_decode, e4m3_encode, wht

GROUP = 16
LEVELS = 16

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


def lloyd_max_normal(n: int = LEVELS, iters: int = 20000) -> np.ndarray:
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


def codebook_f32() -> np.ndarray:
    """The levels as the format stores and uses them (fp32)."""
    return lloyd_max_normal().astype(np.float32)


def thresholds_f32(levels: np.ndarray) -> np.ndarray:
    """Reading V2: fp32 midpoints of adjacent fp32 levels."""
    lv = np.asarray(levels, dtype=np.float32)
    return ((lv[:-1] + lv[1:]) * np.float32(0.5)).astype(np.float32)


# --------------------------------------------------------------------------- group quantisation


def turbo4_quantize(x: np.ndarray):
    """Rotated values (last axis a multiple of 16) -> (packed indices uint8 [..., n/2],
    E4M3 scale codes uint8 [..., n/16]); readings V2-V4."""
    xf = np.asarray(x, dtype=np.float64).astype(np.float32)
    n = xf.shape[-1]
    assert n % GROUP == 0
    g = xf.reshape(*xf.shape[:-1], n // GROUP, GROUP)
    lv = codebook_f32()
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
    flat = idx.reshape(*xf.shape[:-1], n)
    packed = (flat[..., 0::2] | (flat[..., 1::2] << 4)).astype(np.uint8)
    return packed, sc.astype(np.uint8)


def turbo4_unpack(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., n/2] -> indices [..., n] (reading V4)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    out = np.empty((*p.shape[:-1], 2 * p.shape[-1]), dtype=np.int64)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def turbo4_dequantize(packed: np.ndarray, scales_e4m3: np.ndarray) -> np.ndarray:
    """Stored indices and scales -> float64 rotated values, e4m3(s) * level."""
    idx = turbo4_unpack(packed)
    n = idx.shape[-1]
    lv = codebook_f32().astype(np.float64)
    v = lv[idx].reshape(*idx.shape[:-1], n // GROUP, GROUP)
    s = e4m3_decode(scales_e4m3)
    return (v * s[..., None]).reshape(idx.shape)


# --------------------------------------------------------------------------- attention and layer


def attention_decode_bf16k_turbo4v(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, vs: np.ndarray,
                                   seq_len: int) -> np.ndarray:
    """GQA decode attention with bf16 keys and Turbo4 values: scores of the
    unrotated query against the bf16 keys (scale 1/sqrt(D), softmax over
    [0, seq_len)), weights applied to the dequantised rotated values, the
    output rotated back.

    q: [Hq, D] float64; kc: bf16 [cap, Hkv, D]; vc: uint8 [cap, Hkv, D/2];
    vs: uint8 E4M3 [cap, Hkv, D/16].  Returns [Hq, D] float64.
    """
    Hq, D = q.shape
    Hkv = kc.shape[1]
    rep = Hq // Hkv
    K = bf16_to_f64(kc[:seq_len])
    V = turbo4_dequantize(vc[:seq_len], vs[:seq_len])
    out = np.empty((Hq, D))
    for h in range(Hq):
        g = h // rep
        s = K[:, g, :] @ q[h] / math.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ V[:, g, :]
    return wht(out)


def bf16k_turbo4v_append(kv: dict, pos: int, k: np.ndarray, v: np.ndarray) -> dict:
    """A copy of the cache with row ``pos`` holding k as bf16 and the rotated,
    Turbo4-quantised v ([Hkv, D] float64, unrotated)."""
    out = {name: np.array(a, copy=True) for name, a in kv.items()}
    out["k"][pos] = f64_to_bf16(k)
    out["v"][pos], out["v_scales"][pos] = turbo4_quantize(wht(v))
    return out


def forward_full_attention_bf16k_turbo4v(cfg, layer: dict, kv: dict, inv_freq: np.ndarray,
                                         x_in: np.ndarray, cache_pos: int):
    """One token through one gated full-attention layer with a Bf16K + Turbo4V
    cache (the asymmetric branch of ``forward_full_attention``): the bf16
    layer's steps with the value rotated and quantised on append and the
    attention output rotated back.

    kv: {"k": bf16 [cap, Hkv, D], "v": uint8 [cap, Hkv, D/2],
    "v_scales": uint8 [cap, Hkv, D/16]}.  Returns (x_out float64, new_kv, taps).
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
    new_kv = bf16k_turbo4v_append(kv, cache_pos, kr, v.reshape(Hkv, D))
    attn = attention_decode_bf16k_turbo4v(qr, new_kv["k"], new_kv["v"], new_kv["v_scales"],
                                          cache_pos + 1)
    ga = attn * sigmoid(gate)
    o = as_qm(layer["o_proj"]) @ ga.reshape(-1)
    r = x + o
    x_out, mt = mlp_residual(cfg, layer, r)
    taps = {"x_norm": xn, "q_full": q_full, "k": k, "v": v, "q_norm_out": qr.reshape(-1),
            "k_norm_out": kr.reshape(-1), "attn_out": attn.reshape(-1),
            "gated_attn": ga.reshape(-1), "o": o, "x_resid": r, "x_out": x_out}
    taps.update(mt)
    return x_out, new_kv, taps
