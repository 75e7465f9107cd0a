"""GPU parity of the persistent decode kernel (one cooperative launch per token)
on layers-only plans: the tiny two-layer hybrid at every token (fp32, rel 1e-3),
one 4B GDN layer (bf16 outputs at 2e-2, fp32 state at 1e-3 after 64 steps) and
one 4B full-attention layer from cache position 4096 (KV placement checked).
The layer input is written into the plan's first buffer before each step and
the cache position is read on the device, as in graph replay."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import workloads
from gpu_common import ELEM_BF16, ELEM_F32, TOL_BF16, TOL_F32, check, elem_err, rel, say

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def test_persistent_tiny_stack_16_tokens(rt, gen):
    w = workloads.tiny_stack(gen)
    cfg, kinds = w["cfg"], w["kinds"]
    Ls = [rt.GdnLayerDev(w["layers"][0]), rt.FullLayerDev(w["layers"][1])]
    Ss = [rt.GdnStateDev(w["states"][0]), None]
    kv = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in w["kvs"][1].items()}
    kv["k"][:] = NAN_BF16   # sentinel: a read of an unwritten row poisons the output
    kv["v"][:] = NAN_BF16
    KVs = [None, rt.KvCacheDev(kv)]
    inv = rt.inv_freq_dev(cfg)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("tiny persistent plan")
    plan = rt.DecodePlan(cfg, kinds, Ls, Ss, KVs, inv, pos)
    assert plan.n_stages == 11 and plan.first_stage == [0, 5, 11]
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    states, kvs = list(w["states"]), [None, {"k": kv["k"].copy(), "v": kv["v"].copy()}]
    for t, x in enumerate(w["xs"]):
        say(f"tiny persistent token {t}")
        plan.layer_input(0).copy_(rt.to_dev(x))
        pos.fill_(t)
        plan.step()
        torch.cuda.synchronize()
        x1 = O.forward_linear_attention(cfg, w["layers"][0], states[0], x)
        ox, _, states, kvs = O.decode_stack_step(cfg, kinds, w["layers"], states, kvs, inv_h, x, t)
        check(rt.act_to_f32(plan.layer_input(1), cfg), x1[0], TOL_F32, ELEM_F32, 24, t)
        check(rt.act_to_f32(plan.layer_input(2), cfg), ox, TOL_F32, ELEM_F32, 24, t)
    assert plan.check() == 0
    assert rel(Ss[0].to_host()["gdn_state"], states[0]["gdn_state"]) < TOL_F32
    assert rel(Ss[0].to_host()["conv1d_state"], states[0]["conv1d_state"]) < 1e-6
    h = KVs[1].to_host()
    for side in ("k", "v"):
        assert rel(O.bf16_to_f64(h[side]), O.bf16_to_f64(kvs[1][side])) < 1e-2


def test_persistent_plan_reports_a_position_past_the_cache(rt, gen):
    """Stepping past a capacity-16 cache: the step at position 16 writes no KV
    row, its attention output is zero, the kernel exits normally and the error
    word carries the position bit (the earlier steps leave it clear)."""
    from hybrid_decode_amd import binding as B
    w = workloads.tiny_stack(gen, steps=1, capacity=16)
    cfg, kinds = w["cfg"], w["kinds"]
    Ls = [rt.GdnLayerDev(w["layers"][0]), rt.FullLayerDev(w["layers"][1])]
    Ss = [rt.GdnStateDev(w["states"][0]), None]
    KVs = [None, rt.KvCacheDev(w["kvs"][1])]
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = rt.DecodePlan(cfg, kinds, Ls, Ss, KVs, rt.inv_freq_dev(cfg), pos)
    x = rt.to_dev(w["xs"][0])
    for p in (14, 15):
        say(f"persistent step at position {p} of 16")
        plan.layer_input(0).copy_(x)
        pos.fill_(p)
        plan.step()
        torch.cuda.synchronize()
    assert plan.check() == 0
    before = KVs[1].to_host()
    say("persistent step at position 16 of 16")
    plan.layer_input(0).copy_(x)
    pos.fill_(16)
    plan.step()
    torch.cuda.synchronize()
    assert plan.check() == B.Q35_STATUS_POS_RANGE
    after = KVs[1].to_host()
    assert np.array_equal(after["k"], before["k"]) and np.array_equal(after["v"], before["v"])


def test_persistent_gdn_layer_4b_64_steps_and_state(rt, gen):
    """Config 2 through the persistent kernel (64 of its 256 steps)."""
    steps = 64
    w = workloads.gdn_layer_4b(gen, steps=steps)
    cfg, layer, st = w["cfg"], w["layer"], w["state"]
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(st)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = rt.DecodePlan(cfg, ["gdn"], [L], [S], [None], rt.inv_freq_dev(cfg), pos)
    ost = st
    worst = 0.0
    for t, x in enumerate(w["xs"]):
        if t % 16 == 0:
            say(f"persistent 4B GDN step {t}")
        plan.layer_input(0).copy_(rt.to_dev(x))
        plan.step()
        ox, ost, _ = O.forward_linear_attention(cfg, layer, ost, x)
        torch.cuda.synchronize()
        r = rel(rt.act_to_f32(plan.layer_input(1), cfg), ox)
        worst = max(worst, r)
        assert r < TOL_BF16, (t, r)
        assert elem_err(rt.act_to_f32(plan.layer_input(1), cfg), ox, 8) < ELEM_BF16, t
    gst = S.to_host()
    r_state = rel(gst["gdn_state"], ost["gdn_state"])
    r_conv = rel(gst["conv1d_state"], ost["conv1d_state"])
    say(f"persistent 4B GDN: worst output rel {worst:.2e}; after {steps} steps state rel "
        f"{r_state:.2e}, conv rel {r_conv:.2e}")
    assert r_state < TOL_F32 and r_conv < TOL_F32
    assert plan.check() == 0


def test_persistent_full_layer_4b_64_steps_from_4096(rt, gen):
    """Config 3 through the persistent kernel: outputs, KV placement, no reads of
    rows at or past the current position (NaN sentinels)."""
    steps = 64
    w = workloads.full_layer_4b(gen, steps=steps)
    cfg, layer, kv = w["cfg"], w["layer"], w["kv"]
    start = w["start"]
    kv["k"][start:] = NAN_BF16
    kv["v"][start:] = NAN_BF16
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    pos = torch.tensor([start], dtype=torch.int32, device="cuda")
    plan = rt.DecodePlan(cfg, ["full"], [Ld], [None], [KVd], rt.inv_freq_dev(cfg), pos)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {"k": kv["k"].copy(), "v": kv["v"].copy()}
    worst = 0.0
    for i, x in enumerate(w["xs"]):
        t = start + i
        if i % 16 == 0:
            say(f"persistent 4B full attention at cache_pos {t}")
        plan.layer_input(0).copy_(rt.to_dev(x))
        pos.fill_(t)
        plan.step()
        ox, okv, _ = O.forward_full_attention(cfg, layer, okv, inv_h, x, t)
        torch.cuda.synchronize()
        r = rel(rt.act_to_f32(plan.layer_input(1), cfg), ox)
        worst = max(worst, r)
        assert r < TOL_BF16, (t, r)
        assert elem_err(rt.act_to_f32(plan.layer_input(1), cfg), ox, 8) < ELEM_BF16, t
    say(f"persistent 4B full attention: worst output rel {worst:.2e}")
    after = KVd.to_host()
    for side in ("k", "v"):
        assert np.array_equal(after[side][:start], kv[side][:start])
        assert np.all(after[side][start + steps:] == NAN_BF16)
        assert rel(O.bf16_to_f64(after[side][start:start + steps]),
                   O.bf16_to_f64(okv[side][start:start + steps])) < TOL_BF16
    assert plan.check() == 0


def test_persistent_plan_rejects_other_shapes(rt, gen):
    from hybrid_decode_amd import binding as B
    cfg = synth.tiny("bf16")   # tiny dims with bf16 activations: not a built shape
    layer = rt.GdnLayerDev(synth.gdn_layer(gen, cfg, "gpu.pshape"))
    S = rt.GdnStateDev(synth.gdn_state(gen, cfg, "gpu.pshape"))
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.Q35Error) as e:
        rt.DecodePlan(cfg, ["gdn"], [layer], [S], [None], rt.inv_freq_dev(cfg), pos)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED
