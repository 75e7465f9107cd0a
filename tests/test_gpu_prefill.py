"""GPU parity of the multi-token prefill against the oracle's token loop.

The prefill runs T tokens through a layer at once (GEMMs on the matrix cores,
the delta rule in chunks of 64, flash-style causal attention); the oracle runs
the same T decode steps one by one.  Sizes span one token, exactly one chunk,
several chunks with a ragged tail, and the 4B shapes.  Tolerances: layer
outputs rel 1e-3 (fp32 activations) or 2e-2 (bf16), the fp32 GDN state rel
1e-3, the conv state at the outputs' bar; KV rows: which rows change is
checked exactly, the values at rel 4e-3 (one bf16 step), and rows
past the prefill are poisoned with NaN so that a read beyond the causal
extent would show.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import TOL_BF16, TOL_F32, rel, say

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def _workspace(B, cs, T):
    n = B.q35_prefill_workspace_bytes(cs, T)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    assert ws.data_ptr() % 256 == 0
    return ws, n


def _rows_rel(gpu, ref):
    return max(rel(g, r) for g, r in zip(gpu, ref))


# --------------------------------------------------------------------------- GEMM


@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (77, 200, 256), (300, 384, 640), (129, 2560, 2560)])
def test_prefill_gemm_matches_float64_on_the_same_f16_operands(rt, gen, m, n, k):
    from hybrid_decode_amd import binding as B
    say(f"prefill GEMM m={m} n={n} k={k}")
    w = gen.quant(f"pf.gemm.{m}.{n}.{k}", n, k)
    x = gen.normal_f32(f"pf.gemm.x.{m}.{k}", (m, k)).astype(np.float16)
    ref = x.astype(np.float64) @ O.dequant(w).astype(np.float16).astype(np.float64).T
    wq = rt.QuantWeightDev(w)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    B.q35_prefill_gemm(rt.kernels(), wq.struct, xd.data_ptr(), m, y.data_ptr(), rt.stream_ptr())
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    # identical f16 operands: only the fp32 order of the sums differs
    assert rel(got, ref) < 1e-5
    assert _rows_rel(got, ref) < 1e-4


# --------------------------------------------------------------------------- GDN layer


def _gdn_run(rt, cfg, layer, st, x):
    from hybrid_decode_amd import binding as B
    T = x.shape[0]
    cs = rt.cfg_struct(cfg)
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(st)
    xin = rt.to_dev(x)
    xout = torch.empty_like(xin)
    ws, n = _workspace(B, cs, T)
    B.q35_prefill_linear_attention(rt.kernels(), cs, L.struct, S.struct, xin.data_ptr(), T,
                                   xout.data_ptr(), ws.data_ptr(), n, rt.stream_ptr())
    torch.cuda.synchronize()
    return rt.act_to_f32(xout, cfg).reshape(T, cfg.hidden), S.to_host()


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 3, 64, 150])
def test_prefill_gdn_tiny(rt, gen, act, T):
    say(f"prefill GDN tiny act={act} T={T}")
    cfg = synth.tiny(act)
    layer = synth.gdn_layer(gen, cfg, "pf.g")
    st = synth.gdn_state(gen, cfg, "pf.g", 0.2, 0.5)
    x = gen.act(f"pf.g.x{T}", (T, cfg.hidden), act)
    out, gst = _gdn_run(rt, cfg, layer, st, x)
    ref, rst, _ = O.prefill.prefill_linear_attention(cfg, layer, st, x)
    tol = TOL_F32 if act == "f32" else TOL_BF16
    assert _rows_rel(out, ref) < tol
    assert rel(gst["gdn_state"], rst["gdn_state"]) < TOL_F32
    assert rel(gst["conv1d_state"], rst["conv1d_state"]) < TOL_F32


def test_prefill_gdn_4b_three_chunks(rt, gen):
    T = 150
    say(f"prefill GDN 4B T={T}")
    cfg = synth.qwen3_5_4b("bf16")
    layer = synth.gdn_layer(gen, cfg, "pf.g4")
    st = synth.gdn_state(gen, cfg, "pf.g4", 0.05, 0.5)
    x = gen.act("pf.g4.x", (T, cfg.hidden), "bf16")
    out, gst = _gdn_run(rt, cfg, layer, st, x)
    ref, rst, _ = O.prefill.prefill_linear_attention(cfg, layer, st, x)
    assert _rows_rel(out, ref) < TOL_BF16
    assert rel(gst["gdn_state"], rst["gdn_state"]) < TOL_F32
    assert rel(gst["conv1d_state"], rst["conv1d_state"]) < TOL_BF16


def test_prefill_gdn_then_decode_continues_the_state(rt, gen):
    cfg = synth.tiny("f32")
    layer = synth.gdn_layer(gen, cfg, "pf.gc")
    st = synth.gdn_state(gen, cfg, "pf.gc", 0.2, 0.5)
    T = 70
    x = gen.act("pf.gc.x", (T + 1, cfg.hidden), "f32")
    say("prefill GDN then one decode step")
    _, gst = _gdn_run(rt, cfg, layer, st, x[:T])
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(gst)
    scr = rt.GdnScratchDev(cfg)
    x_buf = rt.act_empty(cfg, cfg.hidden)
    rt.forward_linear_attention(cfg, L, S, scr, rt.to_dev(x[T]), x_buf)
    torch.cuda.synchronize()
    ref, rst, _ = O.prefill.prefill_linear_attention(cfg, layer, st, x)
    assert rel(rt.act_to_f32(x_buf, cfg), ref[T]) < TOL_F32
    assert rel(S.to_host()["gdn_state"], rst["gdn_state"]) < TOL_F32


# --------------------------------------------------------------------------- full-attention layer


def _full_run(rt, cfg, layer, kv, x, pos):
    from hybrid_decode_amd import binding as B
    T = x.shape[0]
    cs = rt.cfg_struct(cfg)
    L, K = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    inv = torch.from_numpy(O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)).cuda()
    xin = rt.to_dev(x)
    xout = torch.empty_like(xin)
    ws, n = _workspace(B, cs, T)
    B.q35_prefill_full_attention(rt.kernels(), cs, L.struct, K.struct, inv.data_ptr(), xin.data_ptr(), T,
                                 pos, xout.data_ptr(), ws.data_ptr(), n, rt.stream_ptr())
    torch.cuda.synchronize()
    return rt.act_to_f32(xout, cfg).reshape(T, cfg.hidden), K.to_host()


def _check_cache(after, before, ref, pos, T):
    """Only rows [pos, pos + T) change, and they hold the oracle's rows up to the
    projections' f16 rounding (about 2^-11 of a row's scale) plus the bf16 steps
    that rounding can flip: rel 4e-3, one bf16 step."""
    for side in ("k", "v"):
        changed = np.nonzero(np.any((after[side] != before[side]).reshape(after[side].shape[0], -1),
                                    axis=1))[0]
        assert set(changed.tolist()) <= set(range(pos, pos + T)), side
        assert np.array_equal(after[side][:pos], before[side][:pos]), side
        assert np.array_equal(after[side][pos + T:], before[side][pos + T:]), side
        g = O.bf16_to_f64(after[side][pos:pos + T])
        r = O.bf16_to_f64(ref[side][pos:pos + T])
        assert rel(g, r) < 4e-3, side


@pytest.mark.parametrize("pos,T", [(0, 1), (0, 40), (5, 100), (37, 64)])
def test_prefill_full_tiny(rt, gen, pos, T):
    say(f"prefill full tiny pos={pos} T={T}")
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "pf.f")
    cap = pos + T + 16
    kv = synth.kv_cache(gen, cfg, "pf.f", cap, pos)
    kv["k"][pos + T:] = NAN_BF16
    kv["v"][pos + T:] = NAN_BF16
    x = gen.act(f"pf.f.x{T}", (T, cfg.hidden), "f32")
    before = {s: kv[s].copy() for s in ("k", "v")}
    out, after = _full_run(rt, cfg, layer, kv, x, pos)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos)
    assert np.isfinite(out).all()
    assert _rows_rel(out, ref) < TOL_F32
    _check_cache(after, before, rkv, pos, T)


def test_prefill_full_4b_after_4096_cached_rows(rt, gen):
    pos, T = 4096, 100
    say(f"prefill full 4B pos={pos} T={T}")
    cfg = synth.qwen3_5_4b("bf16")
    layer = synth.full_layer(gen, cfg, "pf.f4")
    cap = pos + T + 32
    kv = synth.kv_cache(gen, cfg, "pf.f4", cap, pos)
    kv["k"][pos + T:] = NAN_BF16
    kv["v"][pos + T:] = NAN_BF16
    x = gen.act("pf.f4.x", (T, cfg.hidden), "bf16")
    before = {s: kv[s].copy() for s in ("k", "v")}
    out, after = _full_run(rt, cfg, layer, kv, x, pos)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos)
    assert np.isfinite(out).all()
    assert _rows_rel(out, ref) < TOL_BF16
    _check_cache(after, before, rkv, pos, T)


def test_prefill_full_then_decode_reads_the_prefilled_rows(rt, gen):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "pf.fc")
    pos, T = 3, 50
    cap = pos + T + 8
    kv = synth.kv_cache(gen, cfg, "pf.fc", cap, pos)
    x = gen.act("pf.fc.x", (T + 1, cfg.hidden), "f32")
    say("prefill full then one decode step")
    _, after = _full_run(rt, cfg, layer, kv, x[:T], pos)
    kv2 = dict(kv)
    kv2.update(after)
    L, K = rt.FullLayerDev(layer), rt.KvCacheDev(kv2)
    scr = rt.FullScratchDev(cfg, cap)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    positions = torch.tensor([pos + T], dtype=torch.int32, device="cuda")
    rt.forward_full_attention(cfg, L, scr, K, torch.from_numpy(inv).cuda(), positions,
                              rt.to_dev(x[T]), pos + T)
    torch.cuda.synchronize()
    ref, _, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos)
    assert rel(rt.act_to_f32(scr.t["x_out"], cfg), ref[T]) < TOL_F32


# --------------------------------------------------------------------------- other head shapes


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 1), (128, 2, 2), (256, 2, 1)])
def test_prefill_full_other_head_shapes(rt, gen, D, Hq, Hkv):
    """The attention kernel's other instantiations: head dims 128 and 256 with one,
    two and eight query heads per kv head (blocks of 64 to 512 threads)."""
    from dataclasses import replace
    pos, T = 7, 70
    say(f"prefill full D={D} Hq={Hq} Hkv={Hkv} pos={pos} T={T}")
    cfg = replace(synth.tiny("f32"), head_dim=D, num_heads=Hq, num_kv_heads=Hkv)
    layer = synth.full_layer(gen, cfg, f"pf.fs{D}.{Hq}.{Hkv}")
    cap = pos + T + 8
    kv = synth.kv_cache(gen, cfg, f"pf.fs{D}", cap, pos)
    kv["k"][pos + T:] = NAN_BF16
    kv["v"][pos + T:] = NAN_BF16
    x = gen.act(f"pf.fs.x{D}", (T, cfg.hidden), "f32")
    before = {s: kv[s].copy() for s in ("k", "v")}
    out, after = _full_run(rt, cfg, layer, kv, x, pos)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos)
    assert np.isfinite(out).all()
    assert _rows_rel(out, ref) < TOL_F32
    _check_cache(after, before, rkv, pos, T)


def test_prefill_gdn_head_dim_64(rt, gen):
    from dataclasses import replace
    T = 100
    say(f"prefill GDN dk=dv=64 T={T}")
    cfg = replace(synth.tiny("f32"), k_head_dim_lin=64, v_head_dim_lin=64)
    layer = synth.gdn_layer(gen, cfg, "pf.g64")
    st = synth.gdn_state(gen, cfg, "pf.g64", 0.2, 0.5)
    x = gen.act("pf.g64.x", (T, cfg.hidden), "f32")
    out, gst = _gdn_run(rt, cfg, layer, st, x)
    ref, rst, _ = O.prefill.prefill_linear_attention(cfg, layer, st, x)
    assert _rows_rel(out, ref) < TOL_F32
    assert rel(gst["gdn_state"], rst["gdn_state"]) < TOL_F32
    assert rel(gst["conv1d_state"], rst["conv1d_state"]) < TOL_F32
