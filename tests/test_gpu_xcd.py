"""GPU parity of the XCD-split decode plan (q35_xcd_*): the GDN mixer and the
MLP each in one launch, split over the eight XCDs and joined by per-XCD
counters, the residual carried between launches as a base plus eight partial
sums.  Checked against the oracle: one 4B GDN layer over 64 steps (every
output, the intermediates of the first step, the fp32 state after), one 4B
full-attention layer over 64 steps from cache position 4096 (outputs, KV
placement, NaN sentinels past the position), the 32-layer stack at context
8192 (its last layer's output fed to the oracle's last layer, logits on sampled
rows, the token, the bookkeeping), graph replay against eager execution, the
plan against the per-layer path on one token, and the error word."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import workloads
from gpu_common import ELEM_BF16, TOL_BF16, TOL_F32, TOL_GEMV_F16, TOL_STACK, check, elem_err, rel, say

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def test_xcd_gdn_layer_4b_64_steps_and_state(rt, gen):
    steps = 64
    w = workloads.gdn_layer_4b(gen, steps=steps)
    cfg, layer, st = w["cfg"], w["layer"], w["state"]
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(st)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("XCD plan, one 4B GDN layer")
    plan = rt.XcdPlan(cfg, ["gdn"], [L], [S], [None], rt.inv_freq_dev(cfg), pos)
    H, I = cfg.hidden, cfg.intermediate
    Hv, dv = cfg.num_v_heads_lin, cfg.v_head_dim_lin
    ost = st
    worst = worst_e = 0.0
    for t, x in enumerate(w["xs"]):
        if t % 16 == 0:
            say(f"XCD 4B GDN step {t}")
        plan.layer_input(0).copy_(rt.to_dev(x))
        plan.step()
        ox, ost, taps = O.forward_linear_attention(cfg, layer, ost, x)
        torch.cuda.synchronize()
        r, e = check(rt.act_to_f32(plan.layer_input(1), cfg), ox, TOL_BF16, ELEM_BF16, 8, t)
        worst, worst_e = max(worst, r), max(worst_e, e)
        if t == 0:
            g = lambda name, n: plan.buffer(name, n).cpu().numpy().astype(np.float64)
            assert rel(g("z", Hv * dv), taps["z"]) < TOL_BF16
            assert rel(g("gate", Hv), taps["gate"]) < TOL_BF16
            assert rel(g("beta", Hv), taps["beta"]) < TOL_BF16
            assert rel(g("y", Hv * dv), taps["gdn_y"]) < TOL_BF16
            parts = g("out_parts", 8 * H).reshape(8, H)
            assert rel(parts.sum(0), taps["gdn_out"]) < TOL_BF16
            assert rel(g("x_resid", H), taps["gdn_x_resid"]) < TOL_BF16
            act = g("mlp_act", I)
            ref_act = O.silu(taps["gate_act"]) * taps["up_act"]
            assert rel(act, ref_act) < TOL_BF16
            xin = rt.act_to_f32(plan.buffer("x_in", H, rt.act_dtype(cfg)), cfg)
            assert np.array_equal(xin, O.act_to_f64(x, cfg.act_dtype))
    gst = S.to_host()
    r_state = rel(gst["gdn_state"], ost["gdn_state"])
    r_conv = rel(gst["conv1d_state"], ost["conv1d_state"])
    say(f"XCD 4B GDN: worst output rel {worst:.2e} (element {worst_e:.3f} RMS); after {steps} steps "
        f"state rel {r_state:.2e}, conv rel {r_conv:.2e}")
    assert r_state < TOL_F32 and r_conv < TOL_F32
    assert plan.check() == 0


def test_xcd_full_layer_4b_64_steps_from_4096(rt, gen):
    steps = 64
    w = workloads.full_layer_4b(gen, steps=steps)
    cfg, layer, kv = w["cfg"], w["layer"], w["kv"]
    start = w["start"]
    kv["k"][start:] = NAN_BF16
    kv["v"][start:] = NAN_BF16
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    pos = torch.tensor([start], dtype=torch.int32, device="cuda")
    say("XCD plan, one 4B full-attention layer")
    plan = rt.XcdPlan(cfg, ["full"], [Ld], [None], [KVd], rt.inv_freq_dev(cfg), pos)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {"k": kv["k"].copy(), "v": kv["v"].copy()}
    worst = 0.0
    for i, x in enumerate(w["xs"]):
        t = start + i
        if i % 16 == 0:
            say(f"XCD 4B full attention at cache_pos {t}")
        plan.layer_input(0).copy_(rt.to_dev(x))
        pos.fill_(t)
        plan.step()
        ox, okv, _ = O.forward_full_attention(cfg, layer, okv, inv_h, x, t)
        torch.cuda.synchronize()
        r = rel(rt.act_to_f32(plan.layer_input(1), cfg), ox)
        worst = max(worst, r)
        assert r < TOL_BF16, (t, r)
        assert elem_err(rt.act_to_f32(plan.layer_input(1), cfg), ox, 8) < ELEM_BF16, t
    say(f"XCD 4B full attention: worst output rel {worst:.2e}")
    after = KVd.to_host()
    for side in ("k", "v"):
        assert np.array_equal(after[side][:start], kv[side][:start])
        assert np.all(after[side][start + steps:] == NAN_BF16)
        assert rel(O.bf16_to_f64(after[side][start:start + steps]),
                   O.bf16_to_f64(okv[side][start:start + steps])) < TOL_BF16
    assert plan.check() == 0


def test_xcd_plan_reports_a_position_past_the_cache(rt, gen):
    from hybrid_decode_amd import binding as B
    w = workloads.full_layer_4b(gen, steps=1)
    cfg, layer, kv = w["cfg"], w["layer"], w["kv"]
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    cap = KVd.capacity
    pos = torch.tensor([cap - 1], dtype=torch.int32, device="cuda")
    plan = rt.XcdPlan(cfg, ["full"], [Ld], [None], [KVd], rt.inv_freq_dev(cfg), pos)
    plan.layer_input(0).copy_(rt.to_dev(w["xs"][0]))
    say(f"XCD step at the last cache row {cap - 1}")
    plan.step()
    torch.cuda.synchronize()
    assert plan.check() == 0
    before = KVd.to_host()
    say(f"XCD step at position {cap}, past the cache")
    pos.fill_(cap)
    plan.step()
    torch.cuda.synchronize()
    assert plan.check() == B.Q35_STATUS_POS_RANGE
    after = KVd.to_host()
    assert np.array_equal(after["k"], before["k"]) and np.array_equal(after["v"], before["v"])


def test_xcd_plan_rejects_other_shapes(rt, gen):
    from hybrid_decode_amd import binding as B
    cfg = synth.tiny("bf16")
    layer = rt.GdnLayerDev(synth.gdn_layer(gen, cfg, "gpu.xshape"))
    S = rt.GdnStateDev(synth.gdn_state(gen, cfg, "gpu.xshape"))
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.Q35Error) as e:
        rt.XcdPlan(cfg, ["gdn"], [layer], [S], [None], rt.inv_freq_dev(cfg), pos)
    assert e.value.status == B.Q35_ERR_UNSUPPORTED


# --------------------------------------------------------------------------- the 32-layer stack


def _snapshot(st):
    return ([None if s is None else (s.conv1d_state.clone(), s.gdn_state.clone()) for s in st.states],
            [None if kv is None else (kv.k.clone(), kv.v.clone()) for kv in st.kvs],
            st.positions.clone(), st.tokens.clone(), st.plan.layer_input(0).clone())


def _restore(st, snap):
    ss, kk, p, t, x0 = snap
    st.plan.layer_input(0).copy_(x0)
    for s, v in zip(st.states, ss):
        if s is not None:
            s.conv1d_state.copy_(v[0])
            s.gdn_state.copy_(v[1])
    for kv, v in zip(st.kvs, kk):
        if kv is not None:
            kv.k.copy_(v[0])
            kv.v.copy_(v[1])
    st.positions.copy_(p)
    st.tokens.copy_(t)
    st.history.fill_(-1)


@pytest.fixture(scope="module")
def xstack8k(rt):
    say("generating the 32-layer 4B stack at ctx 8192 (XCD plan)")
    w = workloads.stack_4b(synth.Gen(0), num_layers=32, ctx=8192, extra=64)
    st = rt.DecodeStack(w["cfg"], w["kinds"], w["layers"], w["states"], w["kvs"], w["embed"],
                        w["final_norm"], w["lm_head"], start_pos=w["ctx"],
                        start_token=w["start_token"], history_len=64, xcd=True)
    torch.cuda.synchronize()
    return w, st


def test_xcd_stack_4b_ctx8192_last_layer_logits_and_token(rt, xstack8k):
    """One token through the plan: the last layer's output checked against the
    oracle's stack evaluated from the same token and the same states and caches
    (32 layers apart: the stack tolerance), the lm_head on sampled rows of the GPU's final
    residual, the token and the bookkeeping."""
    w, st = xstack8k
    cfg, kinds = w["cfg"], w["kinds"]
    plan = st.plan
    snap = _snapshot(st)
    assert np.array_equal(rt.act_to_host(plan.layer_input(0), cfg), w["embed"][w["start_token"]])
    say("one XCD-plan decode step")
    st.step()
    torch.cuda.synchronize()
    assert plan.check() == 0
    pos = w["ctx"]
    x_last = rt.act_to_host(plan.layer_input(len(kinds)), cfg).copy()
    say("oracle stack from the same token")
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    ox, _, _, _ = O.decode_stack_step(cfg, kinds, w["layers"], list(w["states"]), list(w["kvs"]), inv_h,
                                      w["embed"][w["start_token"]], pos)
    r = rel(O.act_to_f64(x_last, "bf16"), ox)
    say(f"stack output rel {r:.2e}")
    assert r < TOL_STACK
    g = st.logits.cpu().numpy()
    tok = int(st.tokens.cpu()[0])
    rows = np.random.default_rng(1).choice(cfg.vocab, 4096, replace=False)
    rows = np.unique(np.concatenate([rows, [tok, int(np.argmax(g))]]))
    h = O.rms_norm(O.act_to_f64(x_last, "bf16"), w["final_norm"], cfg.rms_eps)
    ref = O.dequant({k: v[rows] for k, v in w["lm_head"].items()}).astype(np.float64) @ h
    r = rel(g[rows], ref)
    say(f"sampled logits rel {r:.2e}")
    assert r < TOL_GEMV_F16
    assert tok == int(np.argmax(g))
    assert int(st.positions.cpu()[0]) == pos + 1
    assert int(st.history.cpu()[0]) == tok
    assert np.array_equal(rt.act_to_host(plan.layer_input(0), cfg), w["embed"][tok])
    _restore(st, snap)


def test_xcd_stack_matches_the_per_layer_path(rt, xstack8k):
    """One token through the plan and through the per-layer calls from the same
    state: the final residual and the logits agree within the stack tolerance
    (two valid evaluations of the 32 layers: the split's partial sums of eight
    XCDs change the fp32 summation order, carried through bf16 residuals)."""
    w, st = xstack8k
    cfg, kinds = w["cfg"], w["kinds"]
    snap = _snapshot(st)
    st.step()
    torch.cuda.synchronize()
    assert st.plan.check() == 0
    x_plan = rt.act_to_f32(st.plan.layer_input(len(kinds)), cfg).copy()
    lg_plan = st.logits.cpu().numpy().copy()
    _restore(st, snap)
    say("the same token through the per-layer path")
    ref = rt.DecodeStack(cfg, kinds, w["layers"], w["states"], w["kvs"], w["embed"], w["final_norm"],
                         w["lm_head"], start_pos=w["ctx"], start_token=w["start_token"], history_len=64)
    ref.step()
    torch.cuda.synchronize()
    x_ref = rt.act_to_f32(_act_at(rt, ref, cfg), cfg)
    lg_ref = ref.logits.cpu().numpy()
    r_x, r_l = rel(x_plan, x_ref), rel(lg_plan, lg_ref)
    say(f"plan vs per-layer path: final residual rel {r_x:.2e}, logits rel {r_l:.2e}")
    assert r_x < TOL_STACK and r_l < TOL_STACK
    del ref
    _restore(st, snap)


def _act_at(rt, st, cfg):
    """The per-layer stack's last output (the pointer its step returned)."""
    for t in (st.x_main, st.full_scratch.t["x_out"]):
        if t.data_ptr() == st.last_x:
            return t
    raise AssertionError("last output not found")


def test_xcd_graph_replay_matches_eager(rt, xstack8k):
    w, st = xstack8k
    snap = _snapshot(st)
    steps = 4
    say("eager XCD-plan decode of 4 tokens")
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    eager_hist = st.history.cpu().numpy()[:steps].copy()
    eager_logits = st.logits.cpu().numpy().copy()
    eager_state = st.states[0].gdn_state.cpu().numpy().copy()
    eager_k = st.kvs[3].k.cpu().numpy().copy()
    _restore(st, snap)
    say("capturing one XCD-plan step into a HIP graph")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _restore(st, snap)
    with torch.cuda.graph(graph):
        st.step()
    torch.cuda.synchronize()
    _restore(st, snap)
    for i in range(steps):
        say(f"XCD-plan graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
    assert st.plan.check() == 0
    assert np.array_equal(st.history.cpu().numpy()[:steps], eager_hist)
    assert np.array_equal(st.logits.cpu().numpy(), eager_logits)
    assert np.array_equal(st.states[0].gdn_state.cpu().numpy(), eager_state)
    assert np.array_equal(st.kvs[3].k.cpu().numpy(), eager_k)
    _restore(st, snap)
