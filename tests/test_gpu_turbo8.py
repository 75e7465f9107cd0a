"""GPU parity of the Turbo8 KV cache (E4M3 codes with bf16 scales per 16, in the
Walsh-Hadamard basis of a head) against the oracle.

* the E4M3 decoder the attention loop uses: every finite code bit-exact;
* the group quantiser of the append: codes and scales bit-exact on identical
  fp32 inputs, ties and saturation included;
* tiny layer (fp32 activations, 512 prefilled rows, several attention chunks):
  every step's taps and output at rel 1e-3, the stored row placed exactly and
  equal to the oracle's quantisation; attention re-derived from the stored
  cache and the kernel's own query;
* 4B layer (bf16 activations, 4096 prefilled rows, 12 steps): outputs at rel 2e-2,
  placement exact.  Its projections read x rounded to f16 (relative error near
  1e-3), so its stored codes are compared with the oracle's quantisation of the
  kernel's own k and v, and only loosely with the oracle forward's.

The quantised code is decided on a rotated value that the GPU computes in fp32
and the oracle in fp64: the two can straddle a rounding boundary of E4M3 (about
one element in 10^5 here), so the oracle's cache is teacher-forced to the rows
the kernel stored, and the end-to-end output comparison after a step with any
differing code uses the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import turbo8 as T8
import synth
from synth import workloads
from gpu_common import ELEM_BF16, ELEM_F32, TOL_BF16, TOL_F32, check_gated_attention, elem_err, rel, say

pytestmark = pytest.mark.gpu

NAN_E4M3 = 0x7F


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def test_e4m3_decode_table_matches_oracle_bit_exact(rt):
    from hybrid_decode_amd import binding as B
    say("E4M3 decode table")
    out = torch.full((256,), 7.0, dtype=torch.float32, device="cuda")
    B.q35_fp8_e4m3_table(rt.kernels(), out.data_ptr(), rt.stream_ptr())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = T8.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = np.isfinite(ref)
    assert finite.sum() == 254
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))  # -0 for 0x80
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def _quantiser_inputs(gen) -> np.ndarray:
    """Groups of 16 fp32 values: N(0,1) at scales 2^-30..2^20, a zero group, a
    lone nonzero, exact E4M3 ties after the division, groups whose scale rounds
    down (x / scale above 448, saturating), and a group whose scale is an fp32
    subnormal."""
    groups = []
    n = 512
    base = gen.normal_f32("gpu.t8q.base", (n, 16))
    expo = np.floor(gen.uniform_f32("gpu.t8q.expo", (n,), -30.0, 20.0))
    groups.append(base * np.exp2(expo)[:, None].astype(np.float32))
    groups.append(np.zeros((1, 16), np.float32))
    lone = np.zeros((1, 16), np.float32)
    lone[0, 5] = -3.25
    groups.append(lone)
    # ties: scale s = 2^-4 exactly (amax = 448 s), elements at midpoints of
    # adjacent E4M3 values, so x / s is exactly halfway
    s = np.float32(2.0 ** -4)
    mids = [448.0, 2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 15 * 2.0 ** -10, 1.0625, 1.1875,
            1.3125, 248.0, 432.0, 0.5 + 1 / 32, 17 * 2.0 ** -10, 2.0 ** -6 + 2.0 ** -10, 2.5 + 0.125,
            3.0 + 0.125, 12.0 + 0.5]
    t = np.array(mids, np.float64) * float(s)
    groups.append(t.astype(np.float32)[None])
    groups.append((-t).astype(np.float32)[None])
    # amax just above a bf16 step of amax / 448: the scale rounds down
    sat = np.full((1, 16), 0.5, np.float32)
    sat[0, 0] = np.float32(448.0 * (1 + 2.0 ** -8) * 2.0 ** -7)
    sat[0, 1] = -sat[0, 0]
    groups.append(sat)
    tiny = (base[:2] * np.float32(1e-36)).astype(np.float32)
    groups.append(tiny)
    return np.concatenate(groups).astype(np.float32)


def test_turbo8_quantiser_bit_exact(rt, gen):
    from hybrid_decode_amd import binding as B
    x = _quantiser_inputs(gen)
    G = x.shape[0]
    say(f"Turbo8 quantiser over {G} groups")
    xd = rt.to_dev(x.ravel())
    codes = torch.full((G * 16,), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((G,), 0x1234, dtype=torch.int16, device="cuda")
    B.q35_turbo8_quantize(rt.kernels(), xd.data_ptr(), G * 16, codes.data_ptr(), scales.data_ptr(),
                          rt.stream_ptr())
    torch.cuda.synchronize()
    rc, rs = T8.turbo8_quantize(x.astype(np.float64))
    rs = rs.reshape(G)
    gc = codes.cpu().numpy().reshape(G, 16)
    gs = scales.cpu().numpy().view(np.uint16)
    bad = np.nonzero(np.any(gc != rc, axis=1) | (gs != rs))[0]
    assert bad.size == 0, [(int(i), x[i].tolist(), gc[i].tolist(), rc[i].tolist(), int(gs[i]),
                            int(rs[i])) for i in bad[:3]]
    assert not np.any((gc & 0x7F) == NAN_E4M3)


def test_turbo8_quantiser_rejects_bad_sizes(rt):
    from hybrid_decode_amd import binding as B
    x = torch.zeros(32, dtype=torch.float32, device="cuda")
    c = torch.zeros(32, dtype=torch.uint8, device="cuda")
    s = torch.zeros(2, dtype=torch.int16, device="cuda")
    with pytest.raises(B.Q35Error):
        B.q35_turbo8_quantize(rt.kernels(), x.data_ptr(), 24, c.data_ptr(), s.data_ptr(), None)
    with pytest.raises(B.Q35Error):
        B.q35_turbo8_quantize(rt.kernels(), x.data_ptr(), 32, c.data_ptr(), s.data_ptr() + 1, None)
    B.q35_turbo8_quantize(rt.kernels(), x.data_ptr(), 0, c.data_ptr(), s.data_ptr(), None)


FULL_TAPS_PRE = {"x_norm": "x_norm", "q_full": "q_full", "k": "k", "v": "v",
                 "q_norm_out": "q_norm_out", "k_norm_out": "k_norm_out"}
FULL_TAPS_POST = {"attn_out": "attn_out", "gated_attn": "gated_attn", "o": "o",
                  "x_resid": "x_resid", "x_norm2": "x_norm2", "gate_act": "gate_act",
                  "up_act": "up_act"}


def _check_row(after, before, t, scr, cfg, okv):
    """Row t is the only row that changed; it is the oracle's quantisation of
    the kernel's own post-RoPE k and v (the k_norm_out and v taps, rotated in
    fp64), up to flips of one E4M3 step where the fp32 rotation straddles a
    rounding boundary; and it is within 1e-2 of the row the oracle's own
    forward appended.  Returns whether the row equals that oracle row exactly."""
    Hkv, D = cfg.num_kv_heads, cfg.head_dim
    for side in ("k", "v", "k_scales", "v_scales"):
        changed = np.nonzero(np.any(after[side] != before[side], axis=(1, 2)))[0].tolist()
        assert changed == [t], (side, t, changed)
    own = {"k": scr.t["k_norm_out"], "v": scr.t["v"]}
    same = True
    for side in ("k", "v"):
        gc, gs = after[side][t], after[side + "_scales"][t]
        assert not np.any((gc & 0x7F) == NAN_E4M3)
        x = own[side].cpu().numpy().astype(np.float64).reshape(Hkv, D)
        rc, rs = T8.turbo8_quantize(T8.wht(x))
        rs = rs.reshape(gs.shape)
        assert np.all(np.abs(gs.astype(np.int64) - rs.astype(np.int64)) <= 1), (side, t)
        eq = np.repeat(gs == rs, 16, axis=-1)
        a, b = gc[eq].astype(np.int64), rc[eq].astype(np.int64)
        ma, mb = a & 0x7F, b & 0x7F
        adjacent = ((a >> 7) == (b >> 7)) & (np.abs(ma - mb) <= 1) | ((ma <= 1) & (mb <= 1))
        assert np.all(adjacent), (side, t, a[~adjacent][:4], b[~adjacent][:4])
        assert np.mean(a == b) >= 0.99, (side, t)
        g = T8.turbo8_dequantize(gc, gs)
        r = T8.turbo8_dequantize(okv[side][t], okv[side + "_scales"][t])
        assert rel(g, r) < 1e-2, (side, t)
        same &= bool(np.array_equal(gc, okv[side][t]) and np.array_equal(gs, okv[side + "_scales"][t]))
    return same


def test_full_layer_tiny_turbo8_taps_append_and_attention(rt, gen):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "gpu.t8f")
    start, steps = 512, 16
    cap = start + steps + 8
    kv = synth.kv_cache_turbo8(gen, cfg, "gpu.t8f", cap, start)
    kv["k"][start:] = NAN_E4M3   # poison: any read of an unwritten row gives NaN
    kv["v"][start:] = NAN_E4M3
    kv["k_scales"][start:] = 0x3F80
    kv["v_scales"][start:] = 0x3F80
    # the sparse-V gate off on both sides: the layer's taps are compared exactly
    # here (the gate has its own parity test)
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv, sparse_v=0.0)
    scr = rt.FullScratchDev(cfg, cap, taps=True)
    inv = rt.inv_freq_dev(cfg)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    for i in range(steps):
        t = start + i
        say(f"tiny Turbo8 full attention at cache_pos {t}")
        x = gen.act(f"gpu.t8f.x{i}", (cfg.hidden,), "f32")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        before = KVd.to_host()
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), t)
        torch.cuda.synchronize()
        ox, nkv, taps = T8.forward_full_attention_turbo8(cfg, layer, okv, inv_h, x, t, sparse_v=0.0)
        for k, ok in FULL_TAPS_PRE.items():
            assert rel(scr.t[k].cpu().numpy(), taps[ok]) < TOL_F32, (t, k)
        after = KVd.to_host()
        same = _check_row(after, before, t, scr, cfg, nkv)
        tol = TOL_F32 if same else TOL_BF16
        assert rel(rt.act_to_f32(scr.t["x_out"], cfg), ox) < tol, (t, same)
        assert elem_err(rt.act_to_f32(scr.t["x_out"], cfg), ox, 24) < (ELEM_F32 if same else ELEM_BF16), (t, same)
        for k, ok in FULL_TAPS_POST.items():
            assert rel(scr.t[k].cpu().numpy(), taps[ok]) < tol, (t, k, same)
        # attention from the stored cache and the kernel's own query heads
        qk = scr.t["q_norm_out"].cpu().numpy().astype(np.float64).reshape(cfg.num_heads, cfg.head_dim)
        ref = T8.attention_decode_turbo8(qk, after["k"], after["k_scales"], after["v"],
                                         after["v_scales"], t + 1, sparse_v=0.0)
        assert rel(scr.t["attn_out"].cpu().numpy(), ref) < TOL_F32, t
        okv = {k: np.array(v, copy=True) for k, v in after.items()}   # teacher forcing
    say("tiny Turbo8: all steps within tolerance")


def test_full_layer_4b_turbo8_from_4096(rt, gen):
    w = workloads.full_layer_4b_turbo8(gen, steps=12)
    cfg, layer, kv, start = w["cfg"], w["layer"], w["kv"], w["start"]
    cap = kv["k"].shape[0]
    kv["k"][start:] = NAN_E4M3
    kv["v"][start:] = NAN_E4M3
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    scr = rt.FullScratchDev(cfg, cap, taps=True)
    inv = rt.inv_freq_dev(cfg)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    worst = 0.0
    for i, x in enumerate(w["xs"]):
        t = start + i
        if i % 8 == 0:
            say(f"4B Turbo8 full attention at cache_pos {t}")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        before = KVd.to_host()
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), t)
        torch.cuda.synchronize()
        ox, nkv, _ = T8.forward_full_attention_turbo8(cfg, layer, okv, inv_h, x, t)
        after = KVd.to_host()
        _check_row(after, before, t, scr, cfg, nkv)
        r = rel(rt.act_to_f32(scr.t["x_out"], cfg), ox)
        worst = max(worst, r)
        assert r < TOL_BF16, (t, r)
        assert elem_err(rt.act_to_f32(scr.t["x_out"], cfg), ox, 8) < ELEM_BF16, t
        if i == 0:
            qk = scr.t["q_norm_out"].cpu().numpy().astype(np.float64).reshape(cfg.num_heads,
                                                                               cfg.head_dim)
            # the sparse-V gate at its default on both sides: the kernel drops a
            # subset of the oracle's rows, within their weight of the oracle
            ea, ba, nd = check_gated_attention(scr.t["attn_out"].cpu().numpy(), "turbo8", qk, after,
                                               t + 1, KVd.sparse_v, cfg.num_heads // cfg.num_kv_heads,
                                               TOL_F32)
            say(f"4B Turbo8 attention vs oracle on the stored cache: error {ea:.2e} of the norm "
                f"(dropped-weight bound {ba:.2e}, {nd} (row, head) pairs dropped by the oracle)")
        okv = {k: np.array(v, copy=True) for k, v in after.items()}
    say(f"4B Turbo8 full attention: worst output rel {worst:.2e}")


def test_persistent_plan_rejects_turbo8_cache(rt, gen):
    from hybrid_decode_amd import binding as B
    w = workloads.tiny_stack(gen, steps=1, capacity=16)
    kvs = list(w["kvs"])
    kvs[1] = synth.kv_cache_turbo8(gen, w["cfg"], "gpu.t8plan", 16, 0)
    states = [rt.GdnStateDev(s) if s is not None else None for s in w["states"]]
    layers = [rt.GdnLayerDev(l) if k == "gdn" else rt.FullLayerDev(l)
              for k, l in zip(w["kinds"], w["layers"])]
    kvd = [rt.KvCacheDev(kv) if kv is not None else None for kv in kvs]
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.Q35Error) as e:
        rt.DecodePlan(w["cfg"], w["kinds"], layers, states, kvd, rt.inv_freq_dev(w["cfg"]), pos)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED
