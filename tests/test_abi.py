"""The C-ABI library loads, exports what include/q35decode.h declares, and its
host-side logic (config validation, sizes, error paths) behaves.  No compute
call is made: every call here fails validation before any HIP work."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle as O
import synth
from hybrid_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q35decode.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

FAKE_KERNELS = 0x1000  # a non-NULL handle: only the argument checks run before it would be used


@pytest.fixture(scope="module")
def lib():
    from hybrid_decode_amd import build
    if not build.is_built():
        build.build(verbose=False)
    return B.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q35_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    decl = declared_functions()
    assert decl == sorted(B.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_preset_matches_pages(lib):
    gold = json.load(open(os.path.join(GOLDEN, "qwen35_4b_preset.json")))
    c = B.q35_config_qwen3_5_4b()
    for k, v in gold.items():
        if k in ("source", "derived"):
            continue
        assert getattr(c, k) == pytest.approx(v), k
    assert c.act_dtype == B.Q35_ACT_BF16
    B.q35_config_validate(c)


def test_struct_sizes_match_header_layout(lib):
    # 17 4-byte fields; the quantised-weight struct is 3 pointers + 2 u32
    assert ctypes.sizeof(B.Qwen35ForwardConfig) == 17 * 4
    assert ctypes.sizeof(B.Q35QuantWeight) == 32
    assert ctypes.sizeof(B.LayerKvCache) == 48


def test_tiny_config_validates(lib):
    from hybrid_decode_amd.runtime import cfg_struct
    B.q35_config_validate(cfg_struct(synth.tiny("f32")))
    B.q35_config_validate(cfg_struct(synth.tiny("bf16")))


@pytest.mark.parametrize("field,value,status", [
    ("group_size", 32, B.Q35_ERR_UNSUPPORTED),
    ("num_kv_heads", 3, B.Q35_ERR_INVALID_ARG),
    ("head_dim", 96, B.Q35_ERR_UNSUPPORTED),
    ("rotary_dim", 63, B.Q35_ERR_INVALID_ARG),
    ("rotary_dim", 512, B.Q35_ERR_INVALID_ARG),
    ("num_v_heads_lin", 24, B.Q35_ERR_INVALID_ARG),
    ("v_head_dim_lin", 64, B.Q35_ERR_UNSUPPORTED),
    ("conv_kernel_size", 3, B.Q35_ERR_UNSUPPORTED),
    ("act_dtype", 7, B.Q35_ERR_INVALID_ARG),
    ("hidden", 2500, B.Q35_ERR_INVALID_ARG),
    ("intermediate", 9280, B.Q35_ERR_UNSUPPORTED),
    ("rms_eps", 0.0, B.Q35_ERR_INVALID_ARG),
])
def test_config_validation_errors(lib, field, value, status):
    c = B.q35_config_qwen3_5_4b()
    setattr(c, field, value)
    with pytest.raises(B.Q35Error) as e:
        B.q35_config_validate(c)
    assert e.value.status == status
    assert B.q35_last_error()


def test_kv_dtype_names(lib):
    gold = json.load(open(os.path.join(GOLDEN, "kv_cache_formats.json")))
    for i, name in enumerate(gold["names"]):
        assert B.q35_kv_dtype_from_str(name) == i
    with pytest.raises(B.Q35Error) as e:
        B.q35_kv_dtype_from_str("fp8")
    assert e.value.status == B.Q35_ERR_INVALID_ARG
    assert "fp8" in str(e.value)


def test_kv_cache_bytes_follow_the_alloc_table(lib):
    c = B.q35_config_qwen3_5_4b()
    n = 100 * 1024  # max_seq 100, kv_dim 1024
    expect = {  # (k, v, k_scales, v_scales) per the page's LayerKvCache::alloc table
        "bf16": (2 * n, 2 * n, 0, 0), "turbo8": (n, n, n // 8, n // 8),
        "turbo4": (n // 2, n // 2, n // 16, n // 16), "turbo3": (n * 3 // 8, n * 3 // 8, n // 16, n // 16),
        "turbo2": (n // 4, n // 4, n // 16, n // 16), "bf16k_turbo4v": (2 * n, n // 2, 0, n // 16),
        "bf16k_turbo3v": (2 * n, n * 3 // 8, 0, n // 16), "bf16k_turbo2v": (2 * n, n // 4, 0, n // 16),
    }
    for name, sizes in expect.items():
        assert B.q35_kv_cache_bytes(c, B.q35_kv_dtype_from_str(name), 100) == sizes, name
    c.num_kv_heads, c.head_dim = 1, 8  # kv_dim 8: not a multiple of 16
    with pytest.raises(B.Q35Error):
        B.q35_kv_cache_bytes(c, 1, 4)
    assert B.q35_kv_cache_bytes(c, 0, 4) == (64, 64, 0, 0)


def test_workspace_sizes_grow_with_capacity(lib):
    c = B.q35_config_qwen3_5_4b()
    a = B.q35_full_attention_workspace_bytes(c, 4096)
    b = B.q35_full_attention_workspace_bytes(c, 1 << 20)
    assert 0 < a <= b
    assert B.q35_lm_head_workspace_bytes(c) > 0


def test_rope_inv_freq_matches_oracle(lib):
    c = B.q35_config_qwen3_5_4b()
    assert np.array_equal(B.q35_rope_inv_freq(c), O.rope_inv_freq(1e7, 64))


def test_resolve_without_gpu_reports_no_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(B.Q35Error) as e:
        B.q35_kernels_resolve(0)
    assert e.value.status == B.Q35_ERR_NO_DEVICE


def _full_args(cap=16):
    c = B.q35_config_qwen3_5_4b()
    layer = B.FullAttentionLayer()
    scratch = B.FullAttentionScratch()
    kv = B.LayerKvCache(0x10000, 0x20000, cap, 0, None, None)
    return c, layer, scratch, kv


def test_forward_errors_before_any_launch(lib):
    c, layer, scratch, kv = _full_args()
    # NULL kernel handle
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(None, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG
    # cache position beyond capacity, and a sequence length that is not cache_pos + 1
    for pos, L in ((16, 17), (3, 5), (3, 3)):
        with pytest.raises(B.Q35Error) as e:
            B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100,
                                         pos, L, None)
        assert e.value.status == B.Q35_ERR_OUT_OF_RANGE, (pos, L)
    # Turbo8 needs both scale arrays; the other turbo formats are parsed but not implemented
    kv.dtype = B.q35_kv_dtype_from_str("turbo8")
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "k_scales" in str(e.value)
    kv.k_scales = 0x100
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "v_scales" in str(e.value)
    kv.k_scales = None
    # Bf16K + Turbo4V needs the V scales and no K scales
    kv.dtype = B.q35_kv_dtype_from_str("bf16k_turbo4v")
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "v_scales" in str(e.value)
    kv.k_scales, kv.v_scales = 0x100, 0x100
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "K scale" in str(e.value)
    kv.k_scales, kv.v_scales = None, None
    # the symmetric Lloyd-Max formats need both scale arrays, the asymmetric ones V's only
    for name, needs_k in (("turbo4", True), ("turbo3", True), ("turbo2", True),
                          ("bf16k_turbo3v", False), ("bf16k_turbo2v", False)):
        kv.dtype = B.q35_kv_dtype_from_str(name)
        with pytest.raises(B.Q35Error) as e:
            B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4,
                                         None)
        assert e.value.status == B.Q35_ERR_INVALID_ARG, name
        assert ("k_scales" if needs_k else "v_scales") in str(e.value), name
    # an unknown format number
    kv.dtype = 8
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED
    # valid position but NULL weights
    kv.dtype = 0
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_full_attention(FAKE_KERNELS, c, layer, scratch, kv, 0x100, 0x100, 0x100, 3, 4, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG


def test_linear_attention_errors_before_any_launch(lib):
    c = B.q35_config_qwen3_5_4b()
    layer, state, scratch = B.LinearAttentionLayer(), B.LinearAttentionState(), B.LinearAttentionScratch()
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_linear_attention(FAKE_KERNELS, c, layer, state, scratch, 0x100, 0x100, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG
    # misaligned activation pointer
    with pytest.raises(B.Q35Error) as e:
        B.q35_forward_linear_attention(FAKE_KERNELS, c, layer, state, scratch, 0x104, 0x100, None)
    assert "aligned" in str(e.value)


def test_gemv_shape_errors(lib):
    w = B.Q35QuantWeight(0x1000, 0x2000, 0x3000, 3, 2560)  # 3 rows: not a multiple of 2 at K=2560
    with pytest.raises(B.Q35Error) as e:
        B.q35_gemv(FAKE_KERNELS, w, 0x100, 0x100, B.Q35_ACT_F32, None)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED
    w = B.Q35QuantWeight(0x1000, 0x2000, 0x3000, 4, 2496)
    with pytest.raises(B.Q35Error) as e:
        B.q35_gemv(FAKE_KERNELS, w, 0x100, 0x100, B.Q35_ACT_F32, None)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED


def _prefill_layers(head_dim=None):
    c = B.q35_config_qwen3_5_4b()
    if head_dim is not None:
        c.head_dim, c.rotary_dim = head_dim, head_dim // 4
    fake = 0x100000

    def qw(n, k):
        return B.Q35QuantWeight(fake, fake, fake, n, k)
    H, I = c.hidden, c.intermediate
    full = B.FullAttentionLayer(fake, fake, fake, fake, qw(2 * c.num_heads * c.head_dim, H),
                                qw(c.num_kv_heads * c.head_dim, H), qw(c.num_kv_heads * c.head_dim, H),
                                qw(H, c.num_heads * c.head_dim), qw(I, H), qw(I, H), qw(H, I))
    z = c.num_v_heads_lin * c.v_head_dim_lin
    qkv = 2 * c.num_k_heads_lin * c.k_head_dim_lin + z
    lin = B.LinearAttentionLayer(fake, fake, fake, fake, qw(c.num_v_heads_lin, H), qw(c.num_v_heads_lin, H),
                                 qw(qkv, H), qw(z, H), fake, qw(H, z), fake, qw(I, H), qw(I, H), qw(H, I))
    return c, full, lin, fake


def test_prefill_workspace_grows_with_tokens(lib):
    c = B.q35_config_qwen3_5_4b()
    sizes = [B.q35_prefill_workspace_bytes(c, t) for t in (0, 1, 64, 65, 4096)]
    assert sizes[0] == 0 and all(a < b for a, b in zip(sizes, sizes[1:]))
    assert sizes[-1] % 256 == 0


def test_prefill_workspace_holds_the_largest_projection_as_f16(lib):
    """From 4096 tokens the projections dequantise their weights once into the
    workspace: it must hold the largest set one launch reads (the 4B gate/up
    pair, 2 x 9216 x 2560 f16) beyond what the activations need."""
    c = B.q35_config_qwen3_5_4b()
    one = B.q35_prefill_workspace_bytes(c, 1)
    gate_up_f16 = 2 * c.intermediate * c.hidden * 2
    assert one >= gate_up_f16 + (32 << 20)  # plus the split-GEMM partial tiles


def test_prefill_errors_before_any_launch(lib):
    c, full, lin, fake = _prefill_layers()
    st = B.LinearAttentionState(fake, fake)
    kv = B.LayerKvCache(fake, fake, 128, 0, None, None)
    ws_bytes = B.q35_prefill_workspace_bytes(c, 100)
    # zero tokens: nothing to enqueue, so the fake pointers are never used
    B.q35_prefill_linear_attention(FAKE_KERNELS, c, lin, st, fake, 0, fake, fake, ws_bytes, None)
    B.q35_prefill_full_attention(FAKE_KERNELS, c, full, kv, fake, fake, 0, 5, fake, fake, ws_bytes, None)
    # workspace smaller than the token count needs, or misaligned
    with pytest.raises(B.Q35Error) as e:
        B.q35_prefill_linear_attention(FAKE_KERNELS, c, lin, st, fake, 101, fake, fake, ws_bytes, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "workspace" in str(e.value)
    with pytest.raises(B.Q35Error) as e:
        B.q35_prefill_linear_attention(FAKE_KERNELS, c, lin, st, fake, 10, fake, fake + 16, ws_bytes, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "aligned" in str(e.value)
    # rows past the cache
    with pytest.raises(B.Q35Error) as e:
        B.q35_prefill_full_attention(FAKE_KERNELS, c, full, kv, fake, fake, 100, 29, fake, fake, ws_bytes, None)
    assert e.value.status == B.Q35_ERR_OUT_OF_RANGE
    # a quantised cache so long that the per-token path's attention partials
    # exceed the split area (head_dim 64: the batched path covers 128 and 256)
    c64, full64, _, _ = _prefill_layers(head_dim=64)
    kv.dtype = B.q35_kv_dtype_from_str("turbo8")
    kv.k_scales, kv.v_scales = fake, fake
    kv.capacity = 1 << 25  # partials of 16385 chunks: 67 MB at head_dim 64
    with pytest.raises(B.Q35Error) as e:
        B.q35_prefill_full_attention(FAKE_KERNELS, c64, full64, kv, fake, fake, 10, 0, fake, fake,
                                     B.q35_prefill_workspace_bytes(c64, 100), None)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED and "capacity" in str(e.value)
    kv.capacity = 128
    # a NULL weight
    lin.in_proj_z.codes = None
    with pytest.raises(B.Q35Error) as e:
        B.q35_prefill_linear_attention(FAKE_KERNELS, c, lin, st, fake, 10, fake, fake, ws_bytes, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG and "in_proj_z" in str(e.value)


def test_prefill_gemm_shape_errors(lib):
    w = B.Q35QuantWeight(0x1000, 0x2000, 0x3000, 8, 96)  # k not a multiple of 64
    with pytest.raises(B.Q35Error) as e:
        B.q35_prefill_gemm(FAKE_KERNELS, w, 0x100, 4, 0x100, None, 0, None)
    assert e.value.status == B.Q35_ERR_INVALID_ARG
    w = B.Q35QuantWeight(0x1000, 0x2000, 0x3000, 8, 128)
    # a workspace too small or misaligned for the split partial tiles
    for ws, n in ((0x10000, B.PREFILL_GEMM_WORKSPACE_BYTES - 256), (0x10010, B.PREFILL_GEMM_WORKSPACE_BYTES)):
        with pytest.raises(B.Q35Error) as e:
            B.q35_prefill_gemm(FAKE_KERNELS, w, 0x100, 4, 0x100, ws, n, None)
        assert e.value.status == B.Q35_ERR_INVALID_ARG and "workspace" in str(e.value)
    B.q35_prefill_gemm(FAKE_KERNELS, w, 0x100, 0, 0x100, None, 0, None)  # m == 0: nothing enqueued
    B.q35_prefill_gemm(FAKE_KERNELS, w, 0x100, 0, 0x100, 0x10000, B.PREFILL_GEMM_WORKSPACE_BYTES, None)
