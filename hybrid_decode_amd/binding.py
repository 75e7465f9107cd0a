"""ctypes binding of libq35decode.so: the C-ABI declared in include/q35decode.h.

Argument marshalling only.  Every function here has the name of the C entry
point it calls and raises ``Q35Error`` on a non-zero status.  The library is
loaded from this package directory; when it is missing the import fails loudly
(there is no fallback path).
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq35decode.so")

Q35_OK = 0
Q35_ERR_INVALID_ARG = 1
Q35_ERR_UNSUPPORTED = 2
Q35_ERR_OUT_OF_RANGE = 3
Q35_ERR_HIP = 4
Q35_ERR_NO_DEVICE = 5
# q35_prefill_gemm's optional workspace (Q35_PREFILL_GEMM_WORKSPACE_BYTES)
PREFILL_GEMM_WORKSPACE_BYTES = 32 << 20
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "OUT_OF_RANGE", 4: "HIP", 5: "NO_DEVICE"}

Q35_ACT_BF16 = 0
Q35_ACT_F32 = 1

KV_DTYPES = ["bf16", "turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v",
             "bf16k_turbo2v"]
Q35_KV_BF16 = 0
Q35_KV_TURBO8 = 1
Q35_KV_TURBO4 = 2
Q35_KV_TURBO3 = 3
Q35_KV_TURBO2 = 4
Q35_KV_BF16K_TURBO4V = 5
Q35_KV_BF16K_TURBO3V = 6
Q35_KV_BF16K_TURBO2V = 7

# Every symbol include/q35decode.h declares.
EXPORTS = [
    "q35_last_error", "q35_config_qwen3_5_4b", "q35_config_validate", "q35_rope_inv_freq",
    "q35_kernels_resolve", "q35_kernels_release", "q35_kv_dtype_from_str", "q35_kv_cache_bytes",
    "q35_full_attention_workspace_bytes", "q35_forward_full_attention",
    "q35_forward_full_attention_devpos", "q35_forward_linear_attention", "q35_embed_lookup",
    "q35_lm_head_workspace_bytes", "q35_lm_head_argmax", "q35_lm_head_argmax_noalloc",
    "q35_attention_devpos",
    "q35_gate_up_swiglu", "q35_gemv",
    "q35_decode_workspace_bytes", "q35_decode_plan_create", "q35_decode_plan_release",
    "q35_decode_step", "q35_decode_check", "q35_decode_layer_input", "q35_decode_stage_layout",
    "q35_decode_stage_times", "q35_turbo8_quantize", "q35_fp8_e4m3_table",
    "q35_turbo_codebook", "q35_turbo_quantize", "q35_prefill_workspace_bytes",
    "q35_prefill_linear_attention", "q35_prefill_full_attention", "q35_prefill_gemm",
    "q35_xcd_workspace_bytes", "q35_xcd_plan_create", "q35_xcd_plan_release", "q35_xcd_step",
    "q35_xcd_check", "q35_xcd_layer_input", "q35_xcd_buffers",
]

Q35_LAYER_LINEAR = 0
Q35_LAYER_FULL = 1


class Q35Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"q35 {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


# --------------------------------------------------------------------------- structs

class Qwen35ForwardConfig(C.Structure):
    _fields_ = [("hidden", C.c_uint32), ("intermediate", C.c_uint32), ("num_layers", C.c_uint32),
                ("vocab", C.c_uint32), ("group_size", C.c_uint32), ("rms_eps", C.c_float),
                ("num_heads", C.c_uint32), ("num_kv_heads", C.c_uint32), ("head_dim", C.c_uint32),
                ("rope_theta", C.c_float), ("rotary_dim", C.c_uint32),
                ("num_k_heads_lin", C.c_uint32), ("num_v_heads_lin", C.c_uint32),
                ("k_head_dim_lin", C.c_uint32), ("v_head_dim_lin", C.c_uint32),
                ("conv_kernel_size", C.c_uint32), ("act_dtype", C.c_uint32)]


class Q35QuantWeight(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("n", C.c_uint32), ("k", C.c_uint32)]


class LayerKvCache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_uint32),
                ("dtype", C.c_uint32), ("k_scales", C.c_void_p), ("v_scales", C.c_void_p),
                ("sparse_v", C.c_float)]


class FullAttentionLayer(C.Structure):
    _fields_ = [("input_ln", C.c_void_p), ("q_norm", C.c_void_p), ("k_norm", C.c_void_p),
                ("post_ln", C.c_void_p), ("q_proj", Q35QuantWeight), ("k_proj", Q35QuantWeight),
                ("v_proj", Q35QuantWeight), ("o_proj", Q35QuantWeight),
                ("gate_proj", Q35QuantWeight), ("up_proj", Q35QuantWeight),
                ("down_proj", Q35QuantWeight)]


class FullAttentionScratch(C.Structure):
    _fields_ = [("q_full", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("gated_attn", C.c_void_p), ("x_resid", C.c_void_p), ("mlp_act", C.c_void_p),
                ("x_out", C.c_void_p), ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("x_norm", C.c_void_p), ("q_norm_out", C.c_void_p), ("k_norm_out", C.c_void_p),
                ("attn_out", C.c_void_p), ("o", C.c_void_p), ("x_norm2", C.c_void_p),
                ("gate_act", C.c_void_p), ("up_act", C.c_void_p), ("status", C.c_void_p)]


Q35_STATUS_POS_RANGE = 2
Q35_STATUS_XCD_MAP = 4


class LinearAttentionLayer(C.Structure):
    _fields_ = [("input_ln", C.c_void_p), ("a_log", C.c_void_p), ("dt_bias", C.c_void_p),
                ("conv1d_weight", C.c_void_p), ("in_proj_a", Q35QuantWeight),
                ("in_proj_b", Q35QuantWeight), ("in_proj_qkv", Q35QuantWeight),
                ("in_proj_z", Q35QuantWeight), ("norm_weight", C.c_void_p),
                ("out_proj", Q35QuantWeight), ("post_ln", C.c_void_p),
                ("gate_proj", Q35QuantWeight), ("up_proj", Q35QuantWeight),
                ("down_proj", Q35QuantWeight)]


class LinearAttentionState(C.Structure):
    _fields_ = [("conv1d_state", C.c_void_p), ("gdn_state", C.c_void_p)]


class LinearAttentionScratch(C.Structure):
    _fields_ = [("qkv_conv", C.c_void_p), ("z", C.c_void_p), ("gate", C.c_void_p),
                ("beta", C.c_void_p), ("y", C.c_void_p), ("x_resid", C.c_void_p),
                ("mlp_act", C.c_void_p), ("x_norm", C.c_void_p), ("dt_raw", C.c_void_p),
                ("b_raw", C.c_void_p), ("qkv", C.c_void_p), ("qkv_smooth", C.c_void_p),
                ("y_norm", C.c_void_p), ("out", C.c_void_p), ("x_norm2", C.c_void_p),
                ("gate_act", C.c_void_p), ("up_act", C.c_void_p), ("x_final", C.c_void_p)]


class Q35StackLayer(C.Structure):
    _fields_ = [("kind", C.c_uint32), ("linear", C.POINTER(LinearAttentionLayer)),
                ("state", C.POINTER(LinearAttentionState)), ("full", C.POINTER(FullAttentionLayer)),
                ("kv", C.POINTER(LayerKvCache))]


class Q35DecodeStackDesc(C.Structure):
    _fields_ = [("n_layers", C.c_uint32), ("layers", C.POINTER(Q35StackLayer)),
                ("inv_freq", C.c_void_p), ("positions", C.c_void_p),
                ("lm_head", C.POINTER(Q35QuantWeight)), ("final_norm", C.c_void_p),
                ("embed", C.c_void_p), ("tokens", C.c_void_p), ("logits", C.c_void_p),
                ("history", C.c_void_p), ("history_len", C.c_uint32), ("history_base", C.c_int32)]


class Q35XcdBuffers(C.Structure):
    _fields_ = [("x_in", C.c_void_p), ("qkv_conv", C.c_void_p), ("z", C.c_void_p),
                ("gate", C.c_void_p), ("beta", C.c_void_p), ("y", C.c_void_p),
                ("out_parts", C.c_void_p), ("mlp_act", C.c_void_p), ("mlp_parts", C.c_void_p),
                ("x_mid", C.c_void_p), ("x_resid", C.c_void_p)]


DUMP_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_char_p, C.c_void_p, C.c_uint32)

# --------------------------------------------------------------------------- library

_lib = None


def lib():
    """Load libq35decode.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m hybrid_decode_amd.build`")
        L = C.CDLL(LIB_PATH)
        st, P, u32, i32, sz = C.c_int32, C.POINTER, C.c_uint32, C.c_int32, C.c_size_t
        vp = C.c_void_p
        sig = {
            "q35_last_error": (C.c_char_p, []),
            "q35_config_qwen3_5_4b": (st, [P(Qwen35ForwardConfig)]),
            "q35_config_validate": (st, [P(Qwen35ForwardConfig)]),
            "q35_rope_inv_freq": (st, [P(Qwen35ForwardConfig), P(C.c_float)]),
            "q35_kernels_resolve": (st, [C.c_int, P(vp)]),
            "q35_kernels_release": (None, [vp]),
            "q35_kv_dtype_from_str": (st, [C.c_char_p, P(u32)]),
            "q35_kv_cache_bytes": (st, [P(Qwen35ForwardConfig), u32, u32, P(sz), P(sz), P(sz), P(sz)]),
            "q35_full_attention_workspace_bytes": (st, [P(Qwen35ForwardConfig), u32, P(sz)]),
            "q35_forward_full_attention": (st, [vp, P(Qwen35ForwardConfig), P(FullAttentionLayer),
                                                P(FullAttentionScratch), P(LayerKvCache), vp, vp,
                                                vp, u32, u32, vp, P(vp)]),
            "q35_forward_full_attention_devpos": (st, [vp, P(Qwen35ForwardConfig),
                                                       P(FullAttentionLayer), P(FullAttentionScratch),
                                                       P(LayerKvCache), vp, vp, vp, vp, P(vp)]),
            "q35_forward_linear_attention": (st, [vp, P(Qwen35ForwardConfig),
                                                  P(LinearAttentionLayer), P(LinearAttentionState),
                                                  P(LinearAttentionScratch), vp, vp, vp, DUMP_FN,
                                                  vp, P(vp)]),
            "q35_embed_lookup": (st, [vp, P(Qwen35ForwardConfig), vp, vp, vp, vp]),
            "q35_lm_head_workspace_bytes": (st, [P(Qwen35ForwardConfig), P(sz)]),
            "q35_lm_head_argmax": (st, [vp, P(Qwen35ForwardConfig), vp, P(Q35QuantWeight), vp, vp,
                                        vp, sz, vp, vp, vp, u32, i32, vp, vp, vp]),
            "q35_attention_devpos": (st, [vp, P(Qwen35ForwardConfig), P(FullAttentionLayer),
                                          P(FullAttentionScratch), P(LayerKvCache), vp, vp, vp]),
            "q35_lm_head_argmax_noalloc": (st, [vp, P(Qwen35ForwardConfig), vp, P(Q35QuantWeight),
                                                vp, vp, vp, vp, vp, u32, i32, vp, vp, vp]),
            "q35_gate_up_swiglu": (st, [vp, P(Qwen35ForwardConfig), vp, P(Q35QuantWeight),
                                        P(Q35QuantWeight), vp, vp, vp]),
            "q35_gemv": (st, [vp, P(Q35QuantWeight), vp, vp, u32, vp]),
            "q35_decode_workspace_bytes": (st, [vp, P(Qwen35ForwardConfig), P(Q35DecodeStackDesc),
                                                P(sz)]),
            "q35_decode_plan_create": (st, [vp, P(Qwen35ForwardConfig), P(Q35DecodeStackDesc), vp,
                                            sz, P(vp)]),
            "q35_decode_plan_release": (None, [vp]),
            "q35_decode_step": (st, [vp, vp]),
            "q35_decode_check": (st, [vp, P(u32)]),
            "q35_decode_layer_input": (st, [vp, u32, P(vp)]),
            "q35_decode_stage_layout": (st, [vp, P(u32), P(u32)]),
            "q35_decode_stage_times": (st, [vp, P(C.c_uint64), u32, P(C.c_uint64)]),
            "q35_turbo8_quantize": (st, [vp, vp, u32, vp, vp, vp]),
            "q35_fp8_e4m3_table": (st, [vp, vp, vp]),
            "q35_turbo_codebook": (st, [vp, u32, P(C.c_float)]),
            "q35_turbo_quantize": (st, [vp, u32, vp, u32, vp, vp, vp]),
            "q35_prefill_workspace_bytes": (st, [P(Qwen35ForwardConfig), u32, P(sz)]),
            "q35_prefill_linear_attention": (st, [vp, P(Qwen35ForwardConfig), P(LinearAttentionLayer),
                                                  P(LinearAttentionState), vp, u32, vp, vp, sz, vp]),
            "q35_prefill_full_attention": (st, [vp, P(Qwen35ForwardConfig), P(FullAttentionLayer),
                                                P(LayerKvCache), vp, vp, u32, u32, vp, vp, sz, vp]),
            "q35_prefill_gemm": (st, [vp, P(Q35QuantWeight), vp, u32, vp, vp, sz, vp]),
            "q35_xcd_workspace_bytes": (st, [vp, P(Qwen35ForwardConfig), P(Q35DecodeStackDesc), P(sz)]),
            "q35_xcd_plan_create": (st, [vp, P(Qwen35ForwardConfig), P(Q35DecodeStackDesc), vp, sz,
                                         P(vp)]),
            "q35_xcd_plan_release": (None, [vp]),
            "q35_xcd_step": (st, [vp, vp]),
            "q35_xcd_check": (st, [vp, P(u32)]),
            "q35_xcd_layer_input": (st, [vp, u32, P(vp)]),
            "q35_xcd_buffers": (st, [vp, P(Q35XcdBuffers)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != Q35_OK:
        raise Q35Error(status, lib().q35_last_error().decode())


# --------------------------------------------------------------------------- calls (same names)

def q35_last_error() -> str:
    return lib().q35_last_error().decode()


def q35_config_qwen3_5_4b() -> Qwen35ForwardConfig:
    c = Qwen35ForwardConfig()
    _check(lib().q35_config_qwen3_5_4b(C.byref(c)))
    return c


def q35_config_validate(cfg: Qwen35ForwardConfig) -> None:
    _check(lib().q35_config_validate(C.byref(cfg)))


def q35_rope_inv_freq(cfg: Qwen35ForwardConfig):
    import numpy as np
    out = np.zeros(cfg.rotary_dim // 2, np.float32)
    _check(lib().q35_rope_inv_freq(C.byref(cfg), out.ctypes.data_as(C.POINTER(C.c_float))))
    return out


def q35_kernels_resolve(device: int = 0) -> int:
    h = C.c_void_p()
    _check(lib().q35_kernels_resolve(device, C.byref(h)))
    return h.value


def q35_kernels_release(handle: int) -> None:
    lib().q35_kernels_release(handle)


def q35_kv_dtype_from_str(name: str) -> int:
    d = C.c_uint32()
    _check(lib().q35_kv_dtype_from_str(name.encode(), C.byref(d)))
    return d.value


def q35_kv_cache_bytes(cfg, dtype: int, max_seq: int):
    v = [C.c_size_t() for _ in range(4)]
    _check(lib().q35_kv_cache_bytes(C.byref(cfg), dtype, max_seq, *[C.byref(x) for x in v]))
    return tuple(x.value for x in v)


def q35_full_attention_workspace_bytes(cfg, capacity: int) -> int:
    b = C.c_size_t()
    _check(lib().q35_full_attention_workspace_bytes(C.byref(cfg), capacity, C.byref(b)))
    return b.value


def q35_forward_full_attention(kernels, cfg, layer, scratch, kv, inv_freq, positions, x_in,
                               cache_pos, seq_len_attn, stream) -> int:
    out = C.c_void_p()
    _check(lib().q35_forward_full_attention(kernels, C.byref(cfg), C.byref(layer),
                                            C.byref(scratch), C.byref(kv), inv_freq, positions,
                                            x_in, cache_pos, seq_len_attn, stream, C.byref(out)))
    return out.value


def q35_forward_full_attention_devpos(kernels, cfg, layer, scratch, kv, inv_freq, positions, x_in,
                                      stream) -> int:
    out = C.c_void_p()
    _check(lib().q35_forward_full_attention_devpos(kernels, C.byref(cfg), C.byref(layer),
                                                   C.byref(scratch), C.byref(kv), inv_freq,
                                                   positions, x_in, stream, C.byref(out)))
    return out.value


def q35_forward_linear_attention(kernels, cfg, layer, state, scratch, x_in, x_buf, stream,
                                 dump=None, dump_ctx=None) -> int:
    out = C.c_void_p()
    fn = DUMP_FN(dump) if dump is not None else DUMP_FN()
    _check(lib().q35_forward_linear_attention(kernels, C.byref(cfg), C.byref(layer),
                                              C.byref(state), C.byref(scratch), x_in, x_buf,
                                              stream, fn, dump_ctx, C.byref(out)))
    return out.value


def q35_embed_lookup(kernels, cfg, table, tokens, x_out, stream) -> None:
    _check(lib().q35_embed_lookup(kernels, C.byref(cfg), table, tokens, x_out, stream))


def q35_lm_head_workspace_bytes(cfg) -> int:
    b = C.c_size_t()
    _check(lib().q35_lm_head_workspace_bytes(C.byref(cfg), C.byref(b)))
    return b.value


def q35_lm_head_argmax(kernels, cfg, final_norm, lm_head, x, logits, workspace, workspace_bytes,
                       tokens, positions, history, history_len, history_base, embed_table, x_next,
                       stream) -> None:
    _check(lib().q35_lm_head_argmax(kernels, C.byref(cfg), final_norm, C.byref(lm_head), x,
                                    logits, workspace, workspace_bytes, tokens, positions,
                                    history, history_len, history_base, embed_table, x_next,
                                    stream))


def q35_attention_devpos(kernels, cfg, layer, scratch, kv, inv_freq, positions, stream) -> None:
    _check(lib().q35_attention_devpos(kernels, C.byref(cfg), C.byref(layer), C.byref(scratch),
                                      C.byref(kv), inv_freq, positions, stream))


def q35_lm_head_argmax_noalloc(kernels, cfg, final_norm, lm_head, x, logits, tokens, positions,
                               history, history_len, history_base, embed_table, x_next,
                               stream) -> None:
    _check(lib().q35_lm_head_argmax_noalloc(kernels, C.byref(cfg), final_norm, C.byref(lm_head), x,
                                            logits, tokens, positions, history, history_len,
                                            history_base, embed_table, x_next, stream))


def q35_gate_up_swiglu(kernels, cfg, post_ln, gate_proj, up_proj, x_resid, mlp_act, stream) -> None:
    _check(lib().q35_gate_up_swiglu(kernels, C.byref(cfg), post_ln, C.byref(gate_proj),
                                    C.byref(up_proj), x_resid, mlp_act, stream))


def q35_gemv(kernels, w, x, y, act_dtype, stream) -> None:
    _check(lib().q35_gemv(kernels, C.byref(w), x, y, act_dtype, stream))


def q35_decode_workspace_bytes(kernels, cfg, desc) -> int:
    b = C.c_size_t()
    _check(lib().q35_decode_workspace_bytes(kernels, C.byref(cfg), C.byref(desc), C.byref(b)))
    return b.value


def q35_decode_plan_create(kernels, cfg, desc, workspace, workspace_bytes) -> int:
    h = C.c_void_p()
    _check(lib().q35_decode_plan_create(kernels, C.byref(cfg), C.byref(desc), workspace,
                                        workspace_bytes, C.byref(h)))
    return h.value


def q35_decode_plan_release(plan) -> None:
    lib().q35_decode_plan_release(plan)


def q35_decode_step(plan, stream) -> None:
    _check(lib().q35_decode_step(plan, stream))


def q35_decode_check(plan) -> int:
    e = C.c_uint32()
    _check(lib().q35_decode_check(plan, C.byref(e)))
    return e.value


def q35_decode_layer_input(plan, layer: int) -> int:
    x = C.c_void_p()
    _check(lib().q35_decode_layer_input(plan, layer, C.byref(x)))
    return x.value


def q35_decode_stage_layout(plan, n_layers: int):
    n = C.c_uint32()
    first = (C.c_uint32 * (n_layers + 1))()
    _check(lib().q35_decode_stage_layout(plan, C.byref(n), first))
    return n.value, list(first)


def q35_decode_stage_times(plan, n: int):
    import numpy as np
    ticks = np.zeros(n, np.uint64)
    hz = C.c_uint64()
    _check(lib().q35_decode_stage_times(plan, ticks.ctypes.data_as(C.POINTER(C.c_uint64)), n,
                                        C.byref(hz)))
    return ticks, hz.value


def q35_turbo8_quantize(kernels, x, n: int, codes, scales, stream) -> None:
    _check(lib().q35_turbo8_quantize(kernels, x, n, codes, scales, stream))


def q35_fp8_e4m3_table(kernels, out, stream) -> None:
    _check(lib().q35_fp8_e4m3_table(kernels, out, stream))


def q35_turbo_codebook(kernels, bits: int):
    """The library's b-bit Lloyd-Max codebook (2^bits floats, ascending) as a NumPy array."""
    import numpy as np
    out = (C.c_float * 16)()
    _check(lib().q35_turbo_codebook(kernels, bits, out))
    return np.array(out[:1 << bits], dtype=np.float32)


def q35_turbo_quantize(kernels, bits: int, x, n: int, packed, scales, stream) -> None:
    _check(lib().q35_turbo_quantize(kernels, bits, x, n, packed, scales, stream))


def q35_prefill_workspace_bytes(cfg, max_tokens: int) -> int:
    b = C.c_size_t()
    _check(lib().q35_prefill_workspace_bytes(C.byref(cfg), max_tokens, C.byref(b)))
    return b.value


def q35_prefill_linear_attention(kernels, cfg, layer, state, x_in, n_tokens: int, x_out, workspace,
                                 workspace_bytes: int, stream) -> None:
    _check(lib().q35_prefill_linear_attention(kernels, C.byref(cfg), C.byref(layer), C.byref(state),
                                              x_in, n_tokens, x_out, workspace, workspace_bytes,
                                              stream))


def q35_prefill_full_attention(kernels, cfg, layer, kv, inv_freq, x_in, n_tokens: int,
                               cache_pos: int, x_out, workspace, workspace_bytes: int,
                               stream) -> None:
    _check(lib().q35_prefill_full_attention(kernels, C.byref(cfg), C.byref(layer), C.byref(kv),
                                            inv_freq, x_in, n_tokens, cache_pos, x_out, workspace,
                                            workspace_bytes, stream))


def q35_prefill_gemm(kernels, w, x_f16, m: int, y, workspace, workspace_bytes: int, stream) -> None:
    _check(lib().q35_prefill_gemm(kernels, C.byref(w), x_f16, m, y, workspace, workspace_bytes, stream))


def q35_xcd_workspace_bytes(kernels, cfg, desc) -> int:
    b = C.c_size_t()
    _check(lib().q35_xcd_workspace_bytes(kernels, C.byref(cfg), C.byref(desc), C.byref(b)))
    return b.value


def q35_xcd_plan_create(kernels, cfg, desc, workspace, workspace_bytes) -> int:
    h = C.c_void_p()
    _check(lib().q35_xcd_plan_create(kernels, C.byref(cfg), C.byref(desc), workspace, workspace_bytes,
                                     C.byref(h)))
    return h.value


def q35_xcd_plan_release(plan) -> None:
    lib().q35_xcd_plan_release(plan)


def q35_xcd_step(plan, stream) -> None:
    _check(lib().q35_xcd_step(plan, stream))


def q35_xcd_check(plan) -> int:
    e = C.c_uint32()
    _check(lib().q35_xcd_check(plan, C.byref(e)))
    return e.value


def q35_xcd_layer_input(plan, layer: int) -> int:
    x = C.c_void_p()
    _check(lib().q35_xcd_layer_input(plan, layer, C.byref(x)))
    return x.value


def q35_xcd_buffers(plan) -> Q35XcdBuffers:
    b = Q35XcdBuffers()
    _check(lib().q35_xcd_buffers(plan, C.byref(b)))
    return b
