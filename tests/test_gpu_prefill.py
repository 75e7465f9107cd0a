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
from gpu_common import ELEM_BF16, ELEM_F32, TOL_BF16, TOL_F32, elem_err, rel, say

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


def _check_rows(gpu, ref, tol, act, what=""):
    """Per token: the relative L2 bound, and element by element one step of the
    output format at the oracle's value plus ELEM_* times the token's RMS (the
    element-wise gate of the other layer tests).  Returns the worst of each."""
    bits, elem = (24, ELEM_F32) if act == "f32" else (8, ELEM_BF16)
    r = _rows_rel(gpu, ref)
    e = max(elem_err(g, f, bits) for g, f in zip(gpu, ref))
    assert r < tol, (what, "rel", r)
    assert e < elem, (what, "elem", e)
    return r, e


# --------------------------------------------------------------------------- GEMM


def _gemm(rt, wq, x, m, n, split, f16w=False):
    """q35_prefill_gemm of f16 x [m, k] by wq, fp32 out; with `split` it gets the
    workspace that lets it cut a sparse last round of tiles along k, and with
    `f16w` also the room to dequantise W to f16 once before the product."""
    from hybrid_decode_amd import binding as B
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    nb = B.PREFILL_GEMM_WORKSPACE_BYTES + (2 * wq.n * wq.k if f16w else 0)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if split else None
    B.q35_prefill_gemm(rt.kernels(), wq.struct, xd.data_ptr(), m, y.data_ptr(),
                       ws.data_ptr() if split else None, nb if split else 0, rt.stream_ptr())
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (77, 200, 256), (300, 384, 640), (129, 2560, 2560)])
def test_prefill_gemm_matches_float64_on_the_same_f16_operands(rt, gen, m, n, k, split):
    """With the workspace, every shape but the first (one k tile) has at most a
    quarter as many tiles as compute units, so all its tiles run as 4 or 8 k
    ranges."""
    say(f"prefill GEMM m={m} n={n} k={k} split={split}")
    w = gen.quant(f"pf.gemm.{m}.{n}.{k}", n, k)
    x = gen.normal_f32(f"pf.gemm.x.{m}.{k}", (m, k)).astype(np.float16)
    ref = x.astype(np.float64) @ O.dequant(w).astype(np.float16).astype(np.float64).T
    wq = rt.QuantWeightDev(w)
    got = _gemm(rt, wq, x, m, n, split)
    assert np.isfinite(got).all()
    # identical f16 operands: only the fp32 order of the sums differs
    assert rel(got, ref) < 1e-5
    assert _rows_rel(got, ref) < 1e-4
    if split:
        # W dequantised to f16 once, up front: the same f16 values and the same
        # sums in the same order, so the same bits
        assert np.array_equal(_gemm(rt, wq, x, m, n, True, f16w=True), got)


@pytest.mark.parametrize("n,k", [(9216, 2560), (2560, 9216)])
def test_prefill_gemm_4096_rows_at_the_4b_shapes(rt, gen, n, k):
    """The GEMMs of a 4096-token prompt: gate_proj's shape (the benchmark's; 1152
    tiles, a half-full last round on 256 compute units, run whole) and down_proj's
    (320 tiles: the quarter-full last round is cut in four along k).  Sampled
    rows in every row tile and on the tile edges against float64 on the same f16
    operands; the whole output against the launch without a workspace (never
    split), which differs by fp32 rounding only."""
    m = 4096
    say(f"prefill GEMM m={m} n={n} k={k}")
    w = gen.quant(f"pf.gemm.big.{n}", n, k)
    x = (0.5 * gen.normal_f32(f"pf.gemm.big.x{k}", (m, k))).astype(np.float16)
    wq = rt.QuantWeightDev(w)
    got = _gemm(rt, wq, x, m, n, True)
    plain = _gemm(rt, wq, x, m, n, False)
    f16w = _gemm(rt, wq, x, m, n, True, f16w=True)
    assert np.isfinite(got).all() and np.isfinite(plain).all()
    assert np.array_equal(f16w, got), "W as f16 up front must give the same bits"
    rows = np.array(sorted({0, 1, 255, 256, 511, 1023, 1024, 2047, 2048, 3001, 3839, 3840, 4095}
                           | set(range(17, m, 256))))
    ref = x[rows].astype(np.float64) @ O.dequant(w).astype(np.float16).astype(np.float64).T
    assert _rows_rel(got[rows], ref) < 1e-4
    assert _rows_rel(plain[rows], ref) < 1e-4
    assert _rows_rel(got, plain) < 1e-5


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
    _check_rows(out, ref, tol, cfg.act_dtype)
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
    _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
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


def _full_run(rt, cfg, layer, kv, x, pos, sparse_v=None):
    from hybrid_decode_amd import binding as B
    T = x.shape[0]
    cs = rt.cfg_struct(cfg)
    L = rt.FullLayerDev(layer)
    K = rt.KvCacheDev(kv) if sparse_v is None else rt.KvCacheDev(kv, sparse_v=sparse_v)
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
    _check_rows(out, ref, TOL_F32, cfg.act_dtype)
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
    _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
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
    _check_rows(out, ref, TOL_F32, cfg.act_dtype)
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
    _check_rows(out, ref, TOL_F32, cfg.act_dtype)
    assert rel(gst["gdn_state"], rst["gdn_state"]) < TOL_F32
    assert rel(gst["conv1d_state"], rst["conv1d_state"]) < TOL_F32


# --------------------------------------------------------------------------- edge cases


def test_prefill_zero_tokens_changes_nothing(rt, gen):
    """n_tokens == 0 is an empty prompt: the call succeeds and touches neither the
    state, the cache nor x_out."""
    from hybrid_decode_amd import binding as B
    say("prefill with zero tokens")
    cfg = synth.tiny("f32")
    cs = rt.cfg_struct(cfg)
    ws, n = _workspace(B, cs, 1)
    sentinel = torch.full((cfg.hidden,), 7.0, dtype=torch.float32, device="cuda")
    xin = rt.to_dev(gen.act("pf.z.x", (1, cfg.hidden), "f32"))

    layer = synth.gdn_layer(gen, cfg, "pf.z.g")
    st = synth.gdn_state(gen, cfg, "pf.z.g", 0.2, 0.5)
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(st)
    B.q35_prefill_linear_attention(rt.kernels(), cs, L.struct, S.struct, xin.data_ptr(), 0,
                                   sentinel.data_ptr(), ws.data_ptr(), n, rt.stream_ptr())

    layer = synth.full_layer(gen, cfg, "pf.z.f")
    kv = synth.kv_cache(gen, cfg, "pf.z.f", 16, 5)
    Lf, K = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    inv = torch.from_numpy(O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)).cuda()
    B.q35_prefill_full_attention(rt.kernels(), cs, Lf.struct, K.struct, inv.data_ptr(), xin.data_ptr(), 0,
                                 5, sentinel.data_ptr(), ws.data_ptr(), n, rt.stream_ptr())
    torch.cuda.synchronize()
    after = S.to_host()
    for k in ("gdn_state", "conv1d_state"):
        assert np.array_equal(after[k], st[k]), k
    kv_after = K.to_host()
    for s in ("k", "v"):
        assert np.array_equal(kv_after[s], kv[s]), s
    assert bool((sentinel == 7.0).all())


def test_prefill_full_fills_the_cache_to_capacity(rt, gen):
    """cache_pos + n_tokens == capacity: the last row written is the cache's last
    row (the largest prompt a cache takes)."""
    say("prefill full tiny up to the cache capacity")
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "pf.cap")
    pos, T = 24, 40
    kv = synth.kv_cache(gen, cfg, "pf.cap", pos + T, pos)
    x = gen.act("pf.cap.x", (T, cfg.hidden), "f32")
    before = {s: kv[s].copy() for s in ("k", "v")}
    out, after = _full_run(rt, cfg, layer, kv, x, pos)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos)
    _check_rows(out, ref, TOL_F32, cfg.act_dtype)
    _check_cache(after, before, rkv, pos, T)


# --------------------------------------------------------------------------- 4096-token prompts

BIG_T = 4096


# One call of 4096 tokens against two of 2048: the projections split different
# tail tiles along k (the tile count changes with the prompt length), so the two
# differ by the fp32 order of those sums, which can move a bf16 output or cache
# element by one rounding step (2^-8 relative): SPLIT_BF16 = 4e-3; the fp32 GDN
# state only by fp32 rounding.
SPLIT_BF16, SPLIT_F32 = 4e-3, 1e-5


def _split_rel(a, b):
    """Largest row-relative difference, and whether the two are bit-identical."""
    return _rows_rel(a, b), bool(np.array_equal(a, b))


def _dense32(layer):
    """The layer with its quantised matrices as fp32 dense matrices (the oracle's
    fp32 evaluation of large GEMVs), so a 4096-token loop dequantises each once."""
    return {k: (O.QuantMatrix(v, np.float32) if isinstance(v, dict) and "codes" in v else v)
            for k, v in layer.items()}


def test_prefill_gdn_4b_4096_tokens(rt, gen):
    """The benchmark's prompt through one 4B GDN layer (16 row tiles per GEMM, 64
    chunks): all 4096 outputs (bf16 bar) and the final GDN and conv states (fp32
    bar) against the oracle's loop over the 4096 tokens; all 4096 outputs and the
    final state also against the same
    prompt sent as two calls of 2048 tokens (SPLIT_*)."""
    cfg = synth.qwen3_5_4b("bf16")
    layer = synth.gdn_layer(gen, cfg, "pf.big.g")
    st = synth.gdn_state(gen, cfg, "pf.big.g", 0.05, 0.5)
    x = gen.act("pf.big.g.x", (BIG_T, cfg.hidden), "bf16")
    say(f"prefill GDN 4B T={BIG_T} in one call")
    out, gst = _gdn_run(rt, cfg, layer, st, x)
    assert np.isfinite(out).all() and np.isfinite(gst["gdn_state"]).all()
    say(f"prefill GDN 4B T={BIG_T} as two calls of {BIG_T // 2}")
    o1, s1 = _gdn_run(rt, cfg, layer, st, x[:BIG_T // 2])
    o2, s2 = _gdn_run(rt, cfg, layer, s1, x[BIG_T // 2:])
    r_out, same_out = _split_rel(np.concatenate([o1, o2]), out)
    r_st, same_st = _split_rel(s2["gdn_state"], gst["gdn_state"])
    say(f"  split against one call: outputs rel {r_out:.1e} (bit-identical {same_out}), "
        f"state rel {r_st:.1e} (bit-identical {same_st})")
    assert r_out < SPLIT_BF16 and r_st < SPLIT_F32
    assert rel(s2["conv1d_state"], gst["conv1d_state"]) < SPLIT_F32
    say(f"oracle loop over {BIG_T} tokens")
    ref, ost, _ = O.prefill.prefill_linear_attention(cfg, _dense32(layer), st, x)
    r_all, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    r_last = _rows_rel(out[-64:], ref[-64:])
    r_gst = rel(gst["gdn_state"], ost["gdn_state"])
    r_cst = rel(gst["conv1d_state"], ost["conv1d_state"])
    say(f"  against the oracle: outputs rel {r_all:.2e} (last chunk {r_last:.2e}), GDN state rel "
        f"{r_gst:.2e}, conv state rel {r_cst:.2e}")
    # measured on MI355X: outputs 2.0e-3, GDN state 4.6e-4, conv state 2.8e-4
    assert r_all < TOL_BF16 and r_gst < TOL_F32 and r_cst < TOL_F32


def test_prefill_full_4b_4096_tokens(rt, gen):
    """The benchmark's prompt through one 4B full-attention layer from an empty cache
    of exactly 4096 rows (128 query tiles, up to 64 key tiles per tile): all 4096
    outputs and cache rows against the oracle's loop over the 4096 tokens; all 4096
    outputs and the whole cache against two calls of 2048 tokens, the second at
    cache position 2048 (SPLIT_*)."""
    cfg = synth.qwen3_5_4b("bf16")
    layer = synth.full_layer(gen, cfg, "pf.big.f")
    kv = synth.kv_cache(gen, cfg, "pf.big.f", BIG_T, 0)
    x = gen.act("pf.big.f.x", (BIG_T, cfg.hidden), "bf16")
    say(f"prefill full 4B T={BIG_T} in one call")
    out, after = _full_run(rt, cfg, layer, kv, x, 0)
    assert np.isfinite(out).all()
    say(f"prefill full 4B T={BIG_T} as two calls of {BIG_T // 2}")
    o1, kv1 = _full_run(rt, cfg, layer, kv, x[:BIG_T // 2], 0)
    kv_mid = dict(kv)
    kv_mid.update(kv1)
    o2, kv2 = _full_run(rt, cfg, layer, kv_mid, x[BIG_T // 2:], BIG_T // 2)
    r_out, same_out = _split_rel(np.concatenate([o1, o2]), out)
    say(f"  split against one call: outputs rel {r_out:.1e} (bit-identical {same_out})")
    assert r_out < SPLIT_BF16
    for s in ("k", "v"):
        r_kv, same_kv = _split_rel(O.bf16_to_f64(kv2[s]).reshape(BIG_T, -1),
                                   O.bf16_to_f64(after[s]).reshape(BIG_T, -1))
        say(f"  cache {s}: rel {r_kv:.1e} (bit-identical {same_kv})")
        assert r_kv < SPLIT_BF16, s
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    say(f"oracle loop over {BIG_T} tokens")
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, _dense32(layer), kv, inv, x, 0)
    r_all, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    say(f"  against the oracle: outputs rel {r_all:.2e} (last 64 rows {_rows_rel(out[-64:], ref[-64:]):.2e})")
    assert r_all < TOL_BF16
    for s in ("k", "v"):
        g = O.bf16_to_f64(after[s]).reshape(BIG_T, -1)
        r = O.bf16_to_f64(rkv[s]).reshape(BIG_T, -1)
        say(f"  cache {s} against the oracle: rel {_rows_rel(g, r):.2e}")
        assert _rows_rel(g, r) < 4e-3, s


# --------------------------------------------------------------------------- quantised caches

QFORMATS = ["turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]


def _qcache(gen, cfg, fmt, prefix, cap, filled):
    if fmt == "turbo8":
        return synth.kv_cache_turbo8(gen, cfg, prefix, cap, filled)
    return synth.kv_cache_lm(gen, cfg, prefix, cap, filled, fmt)


def _qrows(fmt, kv, side, rows):
    """Dequantised (rotated-basis) rows of one side of a quantised cache, or the
    bf16 keys of an asymmetric format."""
    from oracle import turbo8 as T8, turbo_lm as TL
    if fmt == "turbo8":
        return T8.turbo8_dequantize(kv[side][rows], kv[side + "_scales"][rows])
    kq, bits = TL.FORMATS[fmt]
    if side == "k" and not kq:
        return O.bf16_to_f64(kv["k"][rows])
    return TL.dequantize(kv[side][rows], kv[side + "_scales"][rows], bits)


def _check_qcache(fmt, after, before, ref, pos, T):
    """Only rows [pos, pos + T) change, and each side holds the oracle's rows up
    to the quantisation flips that the projections' f16 rounding can cause
    (one step of a code in a few elements): rel 5e-2 per side."""
    for name, a in after.items():
        if not isinstance(a, np.ndarray) or a.ndim == 0:
            continue
        cap = a.shape[0]
        changed = np.nonzero(np.any((a != before[name]).reshape(cap, -1), axis=1))[0]
        assert set(changed.tolist()) <= set(range(pos, pos + T)), name
    rows = slice(pos, pos + T)
    for side in ("k", "v"):
        r = rel(_qrows(fmt, after, side, rows), _qrows(fmt, ref, side, rows))
        assert r < 5e-2, (fmt, side, r)


@pytest.mark.parametrize("fmt", QFORMATS)
def test_prefill_full_quantised_tiny(rt, gen, fmt):
    """A prompt into a quantised cache (per-token attention, sparse-V off on both
    sides) against the oracle's decode loop of the format."""
    pos, T = 37, 48
    say(f"prefill full tiny into {fmt} pos={pos} T={T}")
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, f"pfq.{fmt}")
    cap = pos + T + 16
    kv = _qcache(gen, cfg, fmt, f"pfq.{fmt}", cap, pos)
    x = gen.act(f"pfq.{fmt}.x", (T, cfg.hidden), "f32")
    before = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    out, after = _full_run(rt, cfg, layer, kv, x, pos, sparse_v=0.0)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt=fmt, sparse_v=0.0)
    assert np.isfinite(out).all()
    r, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    say(f"  {fmt}: worst token rel {r:.2e}")
    assert r < TOL_BF16
    _check_qcache(fmt, after, before, rkv, pos, T)


@pytest.mark.parametrize("fmt", ["turbo8", "bf16k_turbo4v", "turbo2"])
def test_prefill_full_quantised_4b_after_4096_cached_rows(rt, gen, fmt):
    """The 4B layer, a 16-token prompt after 4096 cached rows, the pages' default
    sparse-V threshold on both sides."""
    pos, T = 4096, 16
    say(f"prefill full 4B into {fmt} pos={pos} T={T}")
    cfg = synth.qwen3_5_4b("bf16")
    layer = synth.full_layer(gen, cfg, f"pfq4.{fmt}")
    cap = pos + T + 32
    kv = _qcache(gen, cfg, fmt, f"pfq4.{fmt}", cap, pos)
    x = gen.act(f"pfq4.{fmt}.x", (T, cfg.hidden), "bf16")
    before = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    out, after = _full_run(rt, cfg, layer, kv, x, pos)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    say("  oracle loop")
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, _dense32(layer), kv, inv, x, pos, fmt=fmt)
    assert np.isfinite(out).all()
    r, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    say(f"  {fmt}: worst token rel {r:.2e}")
    assert r < TOL_BF16
    _check_qcache(fmt, after, before, rkv, pos, T)


@pytest.mark.parametrize("fmt,sparse", [(f, 0.0) for f in QFORMATS] + [("turbo8", None), ("turbo4", None)])
@pytest.mark.parametrize("D", [256, 128])
def test_prefill_full_quantised_tiles(rt, gen, fmt, sparse, D):
    """Head dimension 128 and 256 take the batched path: the prompt's rows
    appended as its decode steps would append them, then one causal attention
    of every token over the rows as stored.  70 prompt tokens after 100 cached
    rows (query blocks of 64 / G tokens, the last one ragged; key tiles of 64
    rows, the last one ragged), the sparse-V gate off on both sides or at the
    pages' default on both (None), against the oracle's decode loop of the
    format: the layer outputs within the bf16 bar and the cache rows as in the
    other quantised prompt tests."""
    from dataclasses import replace
    pos, T = 100, 70
    hq, hkv = (16, 4) if D == 256 else (8, 2)
    cfg = replace(synth.tiny("f32"), num_heads=hq, num_kv_heads=hkv, head_dim=D, rotary_dim=D // 4)
    say(f"prefill full into {fmt} tiles D={D} pos={pos} T={T} sparse_v={sparse}")
    layer = synth.full_layer(gen, cfg, f"pfqt.{fmt}.{D}")
    cap = pos + T + 16
    kv = _qcache(gen, cfg, fmt, f"pfqt.{fmt}.{D}", cap, pos)
    x = gen.act(f"pfqt.{fmt}.{D}.x", (T, cfg.hidden), "f32")
    before = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    kw = {} if sparse is None else {"sparse_v": sparse}
    out, after = _full_run(rt, cfg, layer, kv, x, pos, **kw)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt=fmt, **kw)
    assert np.isfinite(out).all()
    r, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    say(f"  {fmt} D={D}: worst token rel {r:.2e}")
    assert r < TOL_BF16
    _check_qcache(fmt, after, before, rkv, pos, T)


@pytest.mark.parametrize("fmt,D,hq,hkv", [("turbo8", 128, 16, 2), ("turbo3", 128, 16, 2),
                                          ("turbo8", 256, 8, 4), ("turbo8", 128, 4, 4)],
                         ids=["turbo8-d128-g8", "turbo3-d128-g8", "turbo8-d256-g2", "turbo8-d128-g1"])
def test_prefill_full_quantised_tiles_other_groups(rt, gen, fmt, D, hq, hkv):
    """The batched path at the other query-group sizes (64 / G prompt tokens per
    block: 8, 32 and 64), 90 tokens after 50 cached rows, the gate at the
    pages' default on both sides, against the oracle's decode loop."""
    from dataclasses import replace
    pos, T = 50, 90
    cfg = replace(synth.tiny("f32"), num_heads=hq, num_kv_heads=hkv, head_dim=D, rotary_dim=D // 4)
    say(f"prefill full into {fmt} tiles D={D} G={hq // hkv} pos={pos} T={T}")
    layer = synth.full_layer(gen, cfg, f"pfqg.{fmt}.{D}.{hq}")
    cap = pos + T + 8
    kv = _qcache(gen, cfg, fmt, f"pfqg.{fmt}.{D}.{hq}", cap, pos)
    x = gen.act(f"pfqg.{fmt}.{D}.{hq}.x", (T, cfg.hidden), "f32")
    before = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    out, after = _full_run(rt, cfg, layer, kv, x, pos)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt=fmt)
    assert np.isfinite(out).all()
    r, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    say(f"  {fmt} D={D} G={hq // hkv}: worst token rel {r:.2e}")
    assert r < TOL_BF16
    _check_qcache(fmt, after, before, rkv, pos, T)


@pytest.mark.parametrize("pos,T", [(0, 1), (0, 64), (63, 1), (63, 65)])
def test_prefill_full_quantised_tiles_edges(rt, gen, pos, T):
    """Edges of the batched path (Turbo8, D 256, G 4): one token into an empty
    cache (one key row), exactly one tile of tokens, one token whose row is
    the last of the first tile, and a prompt whose query blocks straddle the
    tile boundary; against the oracle's decode loop."""
    from dataclasses import replace
    cfg = replace(synth.tiny("f32"), num_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64)
    say(f"prefill full into turbo8 tiles (edges) pos={pos} T={T}")
    layer = synth.full_layer(gen, cfg, f"pfqe.{pos}.{T}")
    cap = pos + T + 3
    kv = _qcache(gen, cfg, "turbo8", f"pfqe.{pos}.{T}", cap, pos)
    x = gen.act(f"pfqe.{pos}.{T}.x", (T, cfg.hidden), "f32")
    before = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    out, after = _full_run(rt, cfg, layer, kv, x, pos, sparse_v=0.0)
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ref, rkv, _ = O.prefill.prefill_full_attention(cfg, layer, kv, inv, x, pos, fmt="turbo8", sparse_v=0.0)
    assert np.isfinite(out).all()
    r, _ = _check_rows(out, ref, TOL_BF16, cfg.act_dtype)
    say(f"  worst token rel {r:.2e}")
    assert r < TOL_BF16
    _check_qcache("turbo8", after, before, rkv, pos, T)
