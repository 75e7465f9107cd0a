"""GPU parity of the Lloyd-Max KV formats against the oracle: the symmetric
Turbo4/3/2 formats (K and V as b-bit indices into a Lloyd-Max codebook with an
E4M3 norm-keeping scale per 16, in the Walsh-Hadamard basis of a head) and the
asymmetric Bf16K + Turbo4V/3V/2V formats (K in bf16).

* the library's codebooks (2, 3 and 4 bits) equal the oracle's, bit for bit
  (each computed on its own side from the definition);
* the group quantiser of the append: packed indices and scales bit-exact on
  identical fp32 inputs, zero groups, saturating and subnormal scales included;
* tiny layer for each format (fp32 activations, 512 prefilled rows, several
  chunks): every step's taps and output at rel 1e-3, the stored row placed
  exactly, each stored side the oracle's quantisation of the kernel's own k or
  v (a bf16 K the bf16 of the kernel's own k); attention re-derived from the
  stored cache and the kernel's own query;
* 4B layer for each format (bf16 activations, 4096 prefilled rows, 12 steps):
  outputs at 2e-2.

An index is decided on a rotated value that the GPU computes in fp32 and the
oracle in fp64: the two can straddle a threshold, so stored rows are compared
with the oracle's quantisation of the kernel's own inputs (up to rare one-step
flips), the oracle's cache is teacher-forced to the stored rows, and the
end-to-end comparison after a step whose row differs from the oracle forward's
uses the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import turbo_lm as TL
from oracle import turbo8 as T8
import synth
from synth import workloads
from gpu_common import ELEM_BF16, ELEM_F32, TOL_BF16, TOL_F32, check_gated_attention, elem_err, rel, say

pytestmark = pytest.mark.gpu

FORMATS = ["turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_matches_oracle_bit_exact(rt, bits):
    from hybrid_decode_amd import binding as B
    say(f"{bits}-bit codebook")
    lib = B.q35_turbo_codebook(rt.kernels(), bits)
    ref = TL.codebook_f32(bits)
    assert lib.dtype == np.float32 and ref.dtype == np.float32 and lib.shape == ref.shape
    assert np.array_equal(lib.view(np.uint32), ref.view(np.uint32))


def _quantiser_inputs(gen) -> np.ndarray:
    n = 512
    base = gen.normal_f32("gpu.t4q.base", (n, 16))
    expo = np.floor(gen.uniform_f32("gpu.t4q.expo", (n,), -12.0, 12.0))
    groups = [base * np.exp2(expo)[:, None].astype(np.float32)]
    groups.append(np.zeros((1, 16), np.float32))
    lone = np.zeros((1, 16), np.float32)
    lone[0, 3] = 2.5
    groups.append(lone)
    groups.append(np.full((1, 16), -0.75, np.float32))                     # all equal
    groups.append((base[:2] * np.float32(3000.0)).astype(np.float32))      # scale saturates at 448
    groups.append((base[2:4] * np.float32(1e-3)).astype(np.float32))       # subnormal E4M3 scales
    uni = gen.uniform_f32("gpu.t4q.uni", (64, 16), -1.0, 1.0)              # non-Gaussian groups
    groups.append(uni)
    return np.concatenate(groups).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantiser_bit_exact(rt, gen, bits):
    from hybrid_decode_amd import binding as B
    x = _quantiser_inputs(gen)
    G = x.shape[0]
    nb = 2 * bits  # bytes of one group's indices
    say(f"{bits}-bit quantiser over {G} groups")
    xd = rt.to_dev(x.ravel())
    packed = torch.full((G * nb,), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((G,), 0xCD, dtype=torch.uint8, device="cuda")
    B.q35_turbo_quantize(rt.kernels(), bits, xd.data_ptr(), G * 16, packed.data_ptr(), scales.data_ptr(),
                         rt.stream_ptr())
    torch.cuda.synchronize()
    rp, rs = TL.quantize(x.astype(np.float64), bits)
    gp = packed.cpu().numpy().reshape(G, nb)
    gs = scales.cpu().numpy()
    rs = rs.reshape(G)
    bad = np.nonzero(np.any(gp != rp, axis=1) | (gs != rs))[0]
    assert bad.size == 0, [(int(i), x[i].tolist(), gp[i].tolist(), rp[i].tolist(), int(gs[i]),
                            int(rs[i])) for i in bad[:3]]


def test_quantiser_rejects_bad_arguments(rt):
    from hybrid_decode_amd import binding as B
    x = torch.zeros(32, dtype=torch.float32, device="cuda")
    p = torch.zeros(32, dtype=torch.uint8, device="cuda")
    s = torch.zeros(4, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.Q35Error):
        B.q35_turbo_quantize(rt.kernels(), 4, x.data_ptr(), 24, p.data_ptr(), s.data_ptr(), None)
    with pytest.raises(B.Q35Error):
        B.q35_turbo_quantize(rt.kernels(), 4, x.data_ptr(), 32, p.data_ptr() + 4, s.data_ptr(), None)
    with pytest.raises(B.Q35Error):
        B.q35_turbo_quantize(rt.kernels(), 5, x.data_ptr(), 32, p.data_ptr(), s.data_ptr(), None)
    B.q35_turbo_quantize(rt.kernels(), 3, x.data_ptr(), 0, p.data_ptr(), s.data_ptr(), None)


FULL_TAPS_PRE = {"x_norm": "x_norm", "q_full": "q_full", "k": "k", "v": "v",
                 "q_norm_out": "q_norm_out", "k_norm_out": "k_norm_out"}
FULL_TAPS_POST = {"attn_out": "attn_out", "gated_attn": "gated_attn", "o": "o",
                  "x_resid": "x_resid", "x_norm2": "x_norm2", "gate_act": "gate_act",
                  "up_act": "up_act"}


def _check_side(after, t, data, scales, x, bits, okv):
    """A quantised side of row t: the oracle's quantisation of the kernel's own
    input (rotated in fp64) up to rare one-step index flips; close to the row
    the oracle forward appended.  Returns whether it equals that row."""
    rp, rsc = TL.quantize(T8.wht(x), bits)
    gi = TL.unpack_indices(after[data][t], bits)
    ri = TL.unpack_indices(rp, bits)
    assert np.all(np.abs(gi - ri) <= 1), (data, t)
    assert np.mean(gi == ri) >= 0.99, (data, t)
    assert np.all(np.abs(after[scales][t].astype(int) - rsc.astype(int)) <= 1), (data, t)
    g = TL.dequantize(after[data][t], after[scales][t], bits)
    r = TL.dequantize(okv[data][t], okv[scales][t], bits)
    assert rel(g, r) < 5e-2, (data, t)
    return bool(np.array_equal(after[data][t], okv[data][t]) and
                np.array_equal(after[scales][t], okv[scales][t]))


def _check_row(fmt, after, before, t, scr, cfg, okv):
    """Row t is the only row that changed, and each side is as the oracle
    stores the kernel's own k and v.  Returns whether the row equals the oracle
    forward's."""
    kq, bits = TL.FORMATS[fmt]
    Hkv, D = cfg.num_kv_heads, cfg.head_dim
    for side in after:
        changed = np.nonzero(np.any((after[side] != before[side]).reshape(after[side].shape[0], -1),
                                    axis=1))[0].tolist()
        assert changed == [t], (side, t, changed)
    kt = scr.t["k_norm_out"].cpu().numpy().astype(np.float64).reshape(Hkv, D)
    vt = scr.t["v"].cpu().numpy().astype(np.float64).reshape(Hkv, D)
    same = _check_side(after, t, "v", "v_scales", vt, bits, okv)
    if kq:
        same &= _check_side(after, t, "k", "k_scales", kt, bits, okv)
    else:
        assert np.array_equal(after["k"][t], O.f64_to_bf16(kt))
        same &= bool(np.array_equal(after["k"][t], okv["k"][t]))
    return same


def _poison(kv, fmt, start):
    """Unwritten rows read as NaN: bf16 keys NaN, quantised sides a NaN scale."""
    kq, _ = TL.FORMATS[fmt]
    if kq:
        kv["k_scales"][start:] = 0x7F
    else:
        kv["k"][start:] = 0x7FC0
    kv["v_scales"][start:] = 0x7F


@pytest.mark.parametrize("fmt", FORMATS)
def test_full_layer_tiny_taps_append_and_attention(rt, gen, fmt):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, f"gpu.lm.{fmt}")
    start, steps = 512, 16
    cap = start + steps + 8
    kv = synth.kv_cache_lm(gen, cfg, f"gpu.lm.{fmt}", cap, start, fmt)
    _poison(kv, fmt, start)
    # the sparse-V gate off on both sides: the layer's taps are compared exactly
    # here (the gate has its own parity test)
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv, sparse_v=0.0)
    scr = rt.FullScratchDev(cfg, cap, taps=True)
    inv = rt.inv_freq_dev(cfg)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    for i in range(steps):
        t = start + i
        say(f"tiny {fmt} full attention at cache_pos {t}")
        x = gen.act(f"gpu.lm.{fmt}.x{i}", (cfg.hidden,), "f32")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        before = KVd.to_host()
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), t)
        torch.cuda.synchronize()
        ox, nkv, taps = TL.forward_full_attention(fmt, cfg, layer, okv, inv_h, x, t, sparse_v=0.0)
        for k, ok in FULL_TAPS_PRE.items():
            assert rel(scr.t[k].cpu().numpy(), taps[ok]) < TOL_F32, (t, k)
        after = KVd.to_host()
        same = _check_row(fmt, after, before, t, scr, cfg, nkv)
        tol = TOL_F32 if same else TOL_BF16
        assert rel(rt.act_to_f32(scr.t["x_out"], cfg), ox) < tol, (t, same)
        assert elem_err(rt.act_to_f32(scr.t["x_out"], cfg), ox, 24) < (ELEM_F32 if same else ELEM_BF16), (t, same)
        for k, ok in FULL_TAPS_POST.items():
            assert rel(scr.t[k].cpu().numpy(), taps[ok]) < tol, (t, k, same)
        qk = scr.t["q_norm_out"].cpu().numpy().astype(np.float64).reshape(cfg.num_heads, cfg.head_dim)
        ref = TL.attention_decode(fmt, qk, after, t + 1, sparse_v=0.0)
        assert rel(scr.t["attn_out"].cpu().numpy(), ref) < TOL_F32, t
        okv = {k: np.array(v, copy=True) for k, v in after.items()}   # teacher forcing
    say(f"tiny {fmt}: all steps within tolerance")


@pytest.mark.parametrize("fmt", FORMATS)
def test_full_layer_4b_from_4096(rt, gen, fmt):
    w = workloads.full_layer_4b_lm(gen, fmt, steps=12)
    cfg, layer, kv, start = w["cfg"], w["layer"], w["kv"], w["start"]
    cap = kv["k"].shape[0]
    _poison(kv, fmt, start)
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    scr = rt.FullScratchDev(cfg, cap, taps=True)
    inv = rt.inv_freq_dev(cfg)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {k: np.array(v, copy=True) for k, v in kv.items() if isinstance(v, np.ndarray)}
    worst = 0.0
    for i, x in enumerate(w["xs"]):
        t = start + i
        if i % 8 == 0:
            say(f"4B {fmt} full attention at cache_pos {t}")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        before = KVd.to_host()
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), t)
        torch.cuda.synchronize()
        ox, nkv, _ = TL.forward_full_attention(fmt, cfg, layer, okv, inv_h, x, t)
        after = KVd.to_host()
        _check_row(fmt, after, before, t, scr, cfg, nkv)
        r = rel(rt.act_to_f32(scr.t["x_out"], cfg), ox)
        worst = max(worst, r)
        assert r < TOL_BF16, (t, r)
        assert elem_err(rt.act_to_f32(scr.t["x_out"], cfg), ox, 8) < ELEM_BF16, t
        if i == 0:
            qk = scr.t["q_norm_out"].cpu().numpy().astype(np.float64).reshape(cfg.num_heads,
                                                                               cfg.head_dim)
            # the sparse-V gate at its default on both sides: the kernel drops a
            # subset of the oracle's rows, within their weight of the oracle
            ea, ba, nd = check_gated_attention(scr.t["attn_out"].cpu().numpy(), fmt, qk, after, t + 1,
                                               KVd.sparse_v, cfg.num_heads // cfg.num_kv_heads, TOL_F32)
            say(f"4B {fmt} attention vs oracle on the stored cache: error {ea:.2e} of the norm "
                f"(dropped-weight bound {ba:.2e}, {nd} (row, head) pairs dropped by the oracle)")
        okv = {k: np.array(v, copy=True) for k, v in after.items()}
    say(f"4B {fmt} full attention: worst output rel {worst:.2e}")


@pytest.mark.parametrize("fmt", ["turbo3", "bf16k_turbo4v"])
def test_persistent_plan_rejects_lloyd_max_caches(rt, gen, fmt):
    from hybrid_decode_amd import binding as B
    w = workloads.tiny_stack(gen, steps=1, capacity=16)
    kvs = list(w["kvs"])
    kvs[1] = synth.kv_cache_lm(gen, w["cfg"], f"gpu.lmplan.{fmt}", 16, 0, fmt)
    states = [rt.GdnStateDev(s) if s is not None else None for s in w["states"]]
    layers = [rt.GdnLayerDev(l) if k == "gdn" else rt.FullLayerDev(l)
              for k, l in zip(w["kinds"], w["layers"])]
    kvd = [rt.KvCacheDev(kv) if kv is not None else None for kv in kvs]
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.Q35Error) as e:
        rt.DecodePlan(w["cfg"], w["kinds"], layers, states, kvd, rt.inv_freq_dev(w["cfg"]), pos)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED
