"""Seeded synthetic inputs for the Qwen3.5 hybrid decode layers.

This module only draws random numbers and packs them into the storage formats
the decode path reads; it contains none of the decode arithmetic.  The CPU
oracle and the GPU path are both fed the arrays made here, so the two always
see the same bytes.

Random streams come from ``synth.c`` (Philox4x32-10, counter-based), keyed by
a tensor name and a run seed: the same (name, seed, shape) always yields the
same bytes, on any machine and thread count.

Recipe (the value distributions of the synthetic workloads):

* quantised weights: w ~ N(0, 0.02) per element, then per 64-wide group along
  the input dimension s = bf16((max-min)/255), b = bf16(min),
  q = clamp(rint((w-b)/s), 0, 255); only (q, s, b) are kept;
* RMSNorm weights: bf16(1 + 0.1*N(0,1)); conv weights: bf16(U(-0.5, 0.5));
* A_log: fp32 U(0, 2); dt_bias: bf16(N(0, 0.5));
* per-step layer inputs and embeddings: N(0,1) rounded to the activation dtype;
* GDN state / conv state / KV prefill: as the workload specifies.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libq35synth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile synth.c into libq35synth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, f64, vp, cp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p, ctypes.c_char_p
        lib.synth_key.argtypes = [cp, u64]
        lib.synth_key.restype = u64
        for fn in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32", "synth_uniform_bf16"):
            getattr(lib, fn).argtypes = [u64, u64, f64, f64, vp]
            getattr(lib, fn).restype = None
        lib.synth_f32_to_bf16.argtypes = [vp, u64, vp]
        lib.synth_quant_g64.argtypes = [u64, u64, u64, f64, vp, vp, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --------------------------------------------------------------------------- config

@dataclass(frozen=True)
class Config:
    """Dimensions of one Qwen3.5 checkpoint plus the activation dtype."""
    hidden: int
    intermediate: int
    num_layers: int
    vocab: int
    group_size: int
    rms_eps: float
    num_heads: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    rotary_dim: int
    num_k_heads_lin: int
    num_v_heads_lin: int
    k_head_dim_lin: int
    v_head_dim_lin: int
    conv_kernel_size: int
    act_dtype: str = "bf16"  # "bf16" | "f32"

    @property
    def q_total(self) -> int:
        return 2 * self.num_heads * self.head_dim

    @property
    def q_only(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def z_dim_lin(self) -> int:
        return self.num_v_heads_lin * self.v_head_dim_lin

    @property
    def qkv_total_lin(self) -> int:
        return 2 * self.num_k_heads_lin * self.k_head_dim_lin + self.z_dim_lin

    @property
    def num_state_heads(self) -> int:
        return self.num_v_heads_lin


def qwen3_5_4b(act_dtype: str = "bf16") -> Config:
    """The Qwen3.5-4B dimensions (mod.rs page, preset constructor)."""
    return Config(hidden=2560, intermediate=9216, num_layers=32, vocab=248_320, group_size=64,
                  rms_eps=1e-6, num_heads=16, num_kv_heads=4, head_dim=256, rope_theta=1e7,
                  rotary_dim=64, num_k_heads_lin=16, num_v_heads_lin=32, k_head_dim_lin=128,
                  v_head_dim_lin=128, conv_kernel_size=4, act_dtype=act_dtype)


def tiny(act_dtype: str = "f32") -> Config:
    """The tiny two-layer hybrid used for fast parity (layer 0 GDN, layer 1 full)."""
    return Config(hidden=256, intermediate=512, num_layers=2, vocab=0, group_size=64,
                  rms_eps=1e-6, num_heads=4, num_kv_heads=2, head_dim=64, rope_theta=1e7,
                  rotary_dim=16, num_k_heads_lin=2, num_v_heads_lin=4, k_head_dim_lin=32,
                  v_head_dim_lin=32, conv_kernel_size=4, act_dtype=act_dtype)


def with_act(cfg: Config, act_dtype: str) -> Config:
    return replace(cfg, act_dtype=act_dtype)


def layer_kinds(num_layers: int) -> list:
    """Synthetic hybrid layer pattern.

    Two layers: layer 0 GDN, layer 1 full attention (the tiny stack).  Otherwise
    every 4th layer (3, 7, 11, ...) is full attention and the rest are GDN.
    """
    if num_layers == 2:
        return ["gdn", "full"]
    return ["full" if (i + 1) % 4 == 0 else "gdn" for i in range(num_layers)]


# --------------------------------------------------------------------------- draws

class Gen:
    """Named, seeded draws.  ``Gen(seed).normal_f32("x", (4,))`` is reproducible."""

    def __init__(self, seed: int = 0):
        self.seed = int(seed)
        self.lib = _load()

    def key(self, name: str) -> int:
        return int(self.lib.synth_key(name.encode(), self.seed))

    def normal_f32(self, name, shape, mean=0.0, std=1.0) -> np.ndarray:
        out = np.empty(shape, np.float32)
        self.lib.synth_normal_f32(self.key(name), out.size, mean, std, _ptr(out))
        return out

    def normal_bf16(self, name, shape, mean=0.0, std=1.0) -> np.ndarray:
        out = np.empty(shape, np.uint16)
        self.lib.synth_normal_bf16(self.key(name), out.size, mean, std, _ptr(out))
        return out

    def uniform_f32(self, name, shape, lo, hi) -> np.ndarray:
        out = np.empty(shape, np.float32)
        self.lib.synth_uniform_f32(self.key(name), out.size, lo, hi, _ptr(out))
        return out

    def uniform_bf16(self, name, shape, lo, hi) -> np.ndarray:
        out = np.empty(shape, np.uint16)
        self.lib.synth_uniform_bf16(self.key(name), out.size, lo, hi, _ptr(out))
        return out

    def quant(self, name, rows, k, std=0.02) -> dict:
        assert k % 64 == 0
        codes = np.empty((rows, k), np.uint8)
        scales = np.empty((rows, k // 64), np.uint16)
        biases = np.empty((rows, k // 64), np.uint16)
        self.lib.synth_quant_g64(self.key(name), rows, k, std, _ptr(codes), _ptr(scales), _ptr(biases))
        return {"codes": codes, "scales": scales, "biases": biases}

    def act(self, name, shape, act_dtype: str, std=1.0) -> np.ndarray:
        """N(0, std) input stored in the activation dtype (bf16 bits as uint16, or fp32)."""
        if act_dtype == "bf16":
            return self.normal_bf16(name, shape, 0.0, std)
        return self.normal_f32(name, shape, 0.0, std)

    def norm_weight(self, name, n) -> np.ndarray:
        return self.normal_bf16(name, (n,), 1.0, 0.1)


def bf16_bits_of(x_f32: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 (RNE), returned as uint16 bits."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().synth_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


# --------------------------------------------------------------------------- layers

def gdn_layer(g: Gen, cfg: Config, prefix: str) -> dict:
    """Weights of one GDN (linear-attention) layer, field names as in the pages."""
    H, I = cfg.hidden, cfg.intermediate
    Hv = cfg.num_v_heads_lin
    return {
        "input_ln": g.norm_weight(prefix + ".input_ln", H),
        "a_log": g.uniform_f32(prefix + ".a_log", (Hv,), 0.0, 2.0),
        "dt_bias": g.normal_bf16(prefix + ".dt_bias", (Hv,), 0.0, 0.5),
        "conv1d_weight": g.uniform_bf16(prefix + ".conv1d_weight",
                                        (cfg.qkv_total_lin, cfg.conv_kernel_size), -0.5, 0.5),
        "in_proj_a": g.quant(prefix + ".in_proj_a", Hv, H),
        "in_proj_b": g.quant(prefix + ".in_proj_b", Hv, H),
        "in_proj_qkv": g.quant(prefix + ".in_proj_qkv", cfg.qkv_total_lin, H),
        "in_proj_z": g.quant(prefix + ".in_proj_z", cfg.z_dim_lin, H),
        "norm_weight": g.norm_weight(prefix + ".norm_weight", cfg.v_head_dim_lin),
        "out_proj": g.quant(prefix + ".out_proj", H, cfg.z_dim_lin),
        "post_ln": g.norm_weight(prefix + ".post_ln", H),
        "gate_proj": g.quant(prefix + ".gate_proj", I, H),
        "up_proj": g.quant(prefix + ".up_proj", I, H),
        "down_proj": g.quant(prefix + ".down_proj", H, I),
    }


def full_layer(g: Gen, cfg: Config, prefix: str) -> dict:
    """Weights of one gated full-attention layer, field names as in the pages."""
    H, I = cfg.hidden, cfg.intermediate
    return {
        "input_ln": g.norm_weight(prefix + ".input_ln", H),
        "q_norm": g.norm_weight(prefix + ".q_norm", cfg.head_dim),
        "k_norm": g.norm_weight(prefix + ".k_norm", cfg.head_dim),
        "post_ln": g.norm_weight(prefix + ".post_ln", H),
        "q_proj": g.quant(prefix + ".q_proj", cfg.q_total, H),
        "k_proj": g.quant(prefix + ".k_proj", cfg.kv_dim, H),
        "v_proj": g.quant(prefix + ".v_proj", cfg.kv_dim, H),
        "o_proj": g.quant(prefix + ".o_proj", H, cfg.q_only),
        "gate_proj": g.quant(prefix + ".gate_proj", I, H),
        "up_proj": g.quant(prefix + ".up_proj", I, H),
        "down_proj": g.quant(prefix + ".down_proj", H, I),
    }


def gdn_state(g: Gen, cfg: Config, prefix: str, gdn_std: float = 0.0, conv_std: float = 0.0) -> dict:
    """conv1d_state fp32 [qkv_total_lin, K] and gdn_state fp32 [Hv, dk, dv]."""
    cshape = (cfg.qkv_total_lin, cfg.conv_kernel_size)
    sshape = (cfg.num_v_heads_lin, cfg.k_head_dim_lin, cfg.v_head_dim_lin)
    conv = g.normal_f32(prefix + ".conv_state", cshape, 0.0, conv_std) if conv_std > 0 \
        else np.zeros(cshape, np.float32)
    gdn = g.normal_f32(prefix + ".gdn_state", sshape, 0.0, gdn_std) if gdn_std > 0 \
        else np.zeros(sshape, np.float32)
    return {"conv1d_state": conv, "gdn_state": gdn}


def kv_cache(g: Gen, cfg: Config, prefix: str, capacity: int, filled: int) -> dict:
    """bf16 caches [capacity, Hkv, D]; rows [0, filled) hold N(0,1), the rest zero."""
    shape = (capacity, cfg.num_kv_heads, cfg.head_dim)
    k = np.zeros(shape, np.uint16)
    v = np.zeros(shape, np.uint16)
    if filled:
        k[:filled] = g.normal_bf16(prefix + ".k_prefill", (filled,) + shape[1:])
        v[:filled] = g.normal_bf16(prefix + ".v_prefill", (filled,) + shape[1:])
    return {"k": k, "v": v, "capacity": capacity}


LM_FORMATS = {"turbo4": (True, 4), "turbo3": (True, 3), "turbo2": (True, 2),
              "bf16k_turbo4v": (False, 4), "bf16k_turbo3v": (False, 3), "bf16k_turbo2v": (False, 2)}


def kv_cache_lm(g: Gen, cfg: Config, prefix: str, capacity: int, filled: int, fmt: str) -> dict:
    """Lloyd-Max format caches (``fmt`` a key of LM_FORMATS).  A quantised side:
    packed indices uint8 [capacity, Hkv, D*bits/8] with every byte drawn
    uniformly and E4M3 scale bytes [capacity, Hkv, D/16] drawn uniformly from the
    codes 0x28-0x3F (0.25 to 1.875); a bf16 K: [capacity, Hkv, D] N(0, 1).
    Rows [0, filled) are drawn, the others zero."""
    kq, bits = LM_FORMATS[fmt]
    Hkv, D = cfg.num_kv_heads, cfg.head_dim
    nb = D * bits // 8
    out = {"v": np.zeros((capacity, Hkv, nb), np.uint8),
           "v_scales": np.zeros((capacity, Hkv, D // 16), np.uint8), "capacity": capacity,
           "kv_dtype": fmt}
    sides = ["v"]
    if kq:
        out["k"] = np.zeros((capacity, Hkv, nb), np.uint8)
        out["k_scales"] = np.zeros((capacity, Hkv, D // 16), np.uint8)
        sides.append("k")
    else:
        out["k"] = np.zeros((capacity, Hkv, D), np.uint16)
        if filled:
            out["k"][:filled] = g.normal_bf16(prefix + ".k_prefill", (filled, Hkv, D))
    if filled:
        for side in sides:
            u = g.uniform_f32(f"{prefix}.{side}_lm{bits}codes", (filled, Hkv, nb), 0.0, 256.0)
            out[side][:filled] = np.minimum(np.floor(u), 255.0).astype(np.uint8)
            u = g.uniform_f32(f"{prefix}.{side}_lm{bits}scales", (filled, Hkv, D // 16), 0.0, 24.0)
            out[side + "_scales"][:filled] = (0x28 + np.minimum(np.floor(u), 23.0)).astype(np.uint8)
    return out


def kv_cache_bf16k_turbo4v(g: Gen, cfg: Config, prefix: str, capacity: int, filled: int) -> dict:
    """Bf16K + Turbo4V caches (``kv_cache_lm`` with that format)."""
    return kv_cache_lm(g, cfg, prefix, capacity, filled, "bf16k_turbo4v")


def kv_cache_turbo8(g: Gen, cfg: Config, prefix: str, capacity: int, filled: int) -> dict:
    """Turbo8 caches: E4M3 codes uint8 [capacity, Hkv, D] and bf16 group scales
    [capacity, Hkv, D/16].  Rows [0, filled) hold codes drawn uniformly from the
    finite codes (0x00-0x7E and 0x80-0xFE, either sign) and scales bf16(U(1e-3,
    1e-2)), so stored values span the whole E4M3 range, up to about 4.5; the
    other rows are zero."""
    Hkv, D = cfg.num_kv_heads, cfg.head_dim
    shape = (capacity, Hkv, D)
    out = {"k": np.zeros(shape, np.uint8), "v": np.zeros(shape, np.uint8),
           "k_scales": np.zeros((capacity, Hkv, D // 16), np.uint16),
           "v_scales": np.zeros((capacity, Hkv, D // 16), np.uint16), "capacity": capacity}
    if filled:
        for side in ("k", "v"):
            u = g.uniform_f32(f"{prefix}.{side}_t8codes", (filled, Hkv, D), 0.0, 254.0)
            c = np.minimum(np.floor(u), 253.0).astype(np.int64)   # 254 finite codes
            out[side][:filled] = np.where(c < 127, c, c + 1).astype(np.uint8)
            out[side + "_scales"][:filled] = g.uniform_bf16(f"{prefix}.{side}_t8scales",
                                                            (filled, Hkv, D // 16), 1e-3, 1e-2)
    return out
