"""GPU parity of the layer loop: the tiny two-layer hybrid at every step, and the
32-layer 4B-shaped stack (real lm_head) at KV context 8192 and 65536, both
through the per-layer kernels replayed from one HIP graph (the benchmark's
launch configuration) and through the persistent decode kernel, on sampled layers (each fed the GPU's own input to that layer),
sampled logits and the greedy token, plus HIP-graph replay against eager
execution and the two paths against each other."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import workloads
from gpu_common import ELEM_BF16, ELEM_F32, TOL_BF16, TOL_F32, TOL_GEMV_F16, TOL_STACK, check, rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def test_tiny_stack_16_tokens(rt, gen):
    w = workloads.tiny_stack(gen)
    cfg, kinds = w["cfg"], w["kinds"]
    L0, L1 = rt.GdnLayerDev(w["layers"][0]), rt.FullLayerDev(w["layers"][1])
    S0, KV1 = rt.GdnStateDev(w["states"][0]), rt.KvCacheDev(w["kvs"][1])
    gs, fs = rt.GdnScratchDev(cfg), rt.FullScratchDev(cfg, KV1.capacity)
    inv = rt.inv_freq_dev(cfg)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    x_mid = rt.act_empty(cfg, cfg.hidden)
    states, kvs = list(w["states"]), list(w["kvs"])
    for t, x in enumerate(w["xs"]):
        say(f"tiny stack token {t}")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        rt.forward_linear_attention(cfg, L0, S0, gs, rt.to_dev(x), x_mid)
        rt.forward_full_attention(cfg, L1, fs, KV1, inv, pos, x_mid, t)
        torch.cuda.synchronize()
        ox, _, states, kvs = O.decode_stack_step(cfg, kinds, w["layers"], states, kvs, inv_h, x, t)
        check(rt.act_to_f32(fs.t["x_out"], cfg), ox, TOL_F32, ELEM_F32, 24, t)
    assert rel(S0.to_host()["gdn_state"], states[0]["gdn_state"]) < TOL_F32


def _stack_from(rt, w, persistent=False):
    st = rt.DecodeStack(w["cfg"], w["kinds"], w["layers"], w["states"], w["kvs"], w["embed"],
                        w["final_norm"], w["lm_head"], start_pos=w["ctx"],
                        start_token=w["start_token"], history_len=64, persistent=persistent)
    torch.cuda.synchronize()
    return st


def _make_stack(rt, ctx, persistent=False):
    say(f"generating the 32-layer 4B stack at ctx {ctx}")
    g = synth.Gen(0)
    w = workloads.stack_4b(g, num_layers=32, ctx=ctx, extra=64)
    return w, _stack_from(rt, w, persistent)


@pytest.fixture(scope="module")
def stack8k(rt):
    """Config 4: 32 layers (8 full attention), KV at 8192 tokens, lm_head 248320."""
    return _make_stack(rt, 8192)


def _kv_arrays(kv):
    return [t for t in (kv.k, kv.v, kv.k_scales, kv.v_scales) if t is not None]


def _snapshot(st):
    return ([None if s is None else (s.conv1d_state.clone(), s.gdn_state.clone()) for s in st.states],
            [None if kv is None else [t.clone() for t in _kv_arrays(kv)] for kv in st.kvs],
            st.positions.clone(), st.tokens.clone(), st.x_embed.clone(),
            None if st.plan is None else st.plan.layer_input(0).clone())


def _restore(st, snap):
    ss, kk, p, t, x, x0 = snap
    if x0 is not None:
        st.plan.layer_input(0).copy_(x0)
    for s, v in zip(st.states, ss):
        if s is not None:
            s.conv1d_state.copy_(v[0])
            s.gdn_state.copy_(v[1])
    for kv, v in zip(st.kvs, kk):
        if kv is not None:
            for arr, saved in zip(_kv_arrays(kv), v):
                arr.copy_(saved)
    st.positions.copy_(p)
    st.tokens.copy_(t)
    st.x_embed.copy_(x)
    st.history.fill_(-1)


def _check_one_token(rt, w, st, sample_layers):
    """Runs one token layer by layer through the C-ABI (the same calls one graph
    replay makes), checks the sampled layers against the oracle fed with the
    GPU's input to that layer, then the lm_head on sampled rows and the token."""
    from hybrid_decode_amd import binding as B
    cfg, kinds = w["cfg"], w["kinds"]
    snap = _snapshot(st)
    assert np.array_equal(rt.act_to_host(st.x_embed, cfg), w["embed"][w["start_token"]])
    s = rt.stream_ptr()
    x = st.x_embed.data_ptr()
    ins, outs = {}, {}
    last = st.x_embed
    for li, kind in enumerate(kinds):
        if li in sample_layers:
            ins[li] = rt.act_to_host(last, cfg).copy()
        if kind == "gdn":
            B.q35_forward_linear_attention(st.k, st.c, st.layers[li].struct, st.states[li].struct,
                                           st.gdn_scratch.struct, x, st.x_main.data_ptr(), s)
            last = st.x_main
        else:
            B.q35_forward_full_attention_devpos(st.k, st.c, st.layers[li].struct,
                                                st.full_scratch.struct, st.kvs[li].struct,
                                                st.inv_freq.data_ptr(), st.positions.data_ptr(), x, s)
            last = st.full_scratch.t["x_out"]
        x = last.data_ptr()
        if li in sample_layers:
            torch.cuda.synchronize()
            outs[li] = rt.act_to_host(last, cfg).copy()
    torch.cuda.synchronize()
    x_last = rt.act_to_host(last, cfg).copy()
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    pos = w["ctx"]
    for li in sample_layers:
        say(f"oracle check of layer {li} ({kinds[li]})")
        if kinds[li] == "gdn":
            ox, _, _ = O.forward_linear_attention(cfg, w["layers"][li], w["states"][li], ins[li])
        elif "k_scales" in w["kvs"][li]:
            from oracle import turbo8 as T8
            ox, _, _ = T8.forward_full_attention_turbo8(cfg, w["layers"][li], w["kvs"][li], inv_h, ins[li], pos)
        else:
            ox, _, _ = O.forward_full_attention(cfg, w["layers"][li], w["kvs"][li], inv_h, ins[li], pos)
        r, e = check(O.act_to_f64(outs[li], "bf16"), ox, TOL_BF16, ELEM_BF16, 8, li)
        say(f"  layer {li}: rel {r:.2e}, element error {e:.3f} RMS")
    say("lm_head on the stack output")
    B.q35_lm_head_argmax(st.k, st.c, st.final_norm.data_ptr(), st.lm_head.struct, x,
                         st.logits.data_ptr(), st.lm_ws.data_ptr(), st.lm_ws.numel(),
                         st.tokens.data_ptr(), st.positions.data_ptr(), st.history.data_ptr(),
                         st.history_len, st.history_base, st.embed.data_ptr(),
                         st.x_embed.data_ptr(), s)
    torch.cuda.synchronize()
    g = st.logits.cpu().numpy()
    rows = np.random.default_rng(0).choice(cfg.vocab, 4096, replace=False)
    tok = int(st.tokens.cpu()[0])
    rows = np.unique(np.concatenate([rows, [tok, int(np.argmax(g))]]))
    h = O.rms_norm(O.act_to_f64(x_last, "bf16"), w["final_norm"], cfg.rms_eps)
    ref = O.dequant({k: v[rows] for k, v in w["lm_head"].items()}).astype(np.float64) @ h
    r = rel(g[rows], ref)
    say(f"sampled logits rel {r:.2e}")
    assert r < TOL_GEMV_F16
    assert tok == int(np.argmax(g))
    assert int(st.positions.cpu()[0]) == pos + 1
    assert int(st.history.cpu()[0]) == tok
    assert np.array_equal(rt.act_to_host(st.x_embed, cfg), w["embed"][tok])
    _restore(st, snap)


def test_stack_4b_ctx8192_sampled_layers_logits_and_token(rt, stack8k):
    w, st = stack8k
    # first GDN, a middle GDN, first / middle / last full attention, last GDN before it
    _check_one_token(rt, w, st, sample_layers=(0, 3, 13, 15, 30, 31))


def test_stack_4b_ctx8192_graph_replay_matches_eager(rt, stack8k):
    _graph_replay_matches_eager(rt, *stack8k)


def test_stack_4b_ctx8192_turbo8_tiles(rt):
    """Config 4 with Turbo8 caches: at capacity 8256 the full-attention layers run
    the matrix-core tiles (72-row chunks, the kv heads of a chunk on one XCD)
    from the device position.  One token layer by layer against the oracle
    (sampled GDN and full-attention layers, each fed the GPU's input; the
    pages' default sparse-V threshold on both sides), the lm_head and the
    token; then graph replays against eager, bit for bit."""
    say("generating the 32-layer 4B stack with Turbo8 caches at ctx 8192")
    w = workloads.stack_4b(synth.Gen(0), num_layers=32, ctx=8192, extra=64, kv="turbo8")
    st = _stack_from(rt, w)
    _check_one_token(rt, w, st, sample_layers=(3, 15, 30, 31))
    _graph_replay_matches_eager(rt, w, st)


def _graph_replay_matches_eager(rt, w, st):
    snap = _snapshot(st)
    steps = 6
    say("eager decode of 6 tokens")
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    eager_hist = st.history.cpu().numpy()[:steps].copy()
    eager_logits = st.logits.cpu().numpy().copy()
    eager_state = st.states[0].gdn_state.cpu().numpy().copy()
    eager_k = [t.cpu().numpy().copy() for t in _kv_arrays(st.kvs[3])]
    assert np.all(eager_hist >= 0)
    _restore(st, snap)
    say("capturing one decode step into a HIP graph")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step()            # warm-up on the capture stream (one real token)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _restore(st, snap)
    with torch.cuda.graph(graph):
        st.step()
    torch.cuda.synchronize()
    _restore(st, snap)   # capture recorded the launches; state is reset before replay
    for i in range(steps):
        say(f"graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
    assert np.array_equal(st.history.cpu().numpy()[:steps], eager_hist)
    assert np.array_equal(st.logits.cpu().numpy(), eager_logits)
    assert np.array_equal(st.states[0].gdn_state.cpu().numpy(), eager_state)
    for arr, e in zip(_kv_arrays(st.kvs[3]), eager_k):
        assert np.array_equal(arr.cpu().numpy(), e)
    _restore(st, snap)


def _oracle_weights(w):
    """The stack's layers with every quantised matrix as an fp32 dense matrix,
    dequantised once (the oracle's fp32 evaluation of stack-sized GEMVs)."""
    ql = lambda l: {k: (O.QuantMatrix(v, np.float32) if isinstance(v, dict) and "codes" in v else v)
                    for k, v in l.items()}
    layers = [ql(l) for l in w["layers"]]
    lm = O.QuantMatrix(w["lm_head"], np.float32)
    for i, l in enumerate(layers):
        for v in l.values():
            if isinstance(v, O.QuantMatrix):
                v.dense()
        if i % 8 == 7:
            say(f"  oracle weights of layer {i} dequantised")
    lm.dense()
    return layers, lm


def test_stack_4b_ctx8192_16_greedy_tokens_teacher_forced(rt, stack8k):
    """Config 4 in the benchmark's launch configuration: 16 greedy tokens from one
    HIP graph per token with no logits stored.  The same token sequence is then
    run layer by layer through the C-ABI with the logits kept (its tokens must
    be the graph's), and checked against the oracle two ways, every step:
    each of the 32 layers fed the GPU's input to that layer (output within the
    bf16 gates), and the whole oracle stack fed the GPU's tokens (its logits
    within TOL_STACK of the GPU's; the same stack evaluated with the pages'
    bf16 buffers rounded, the oracle's Mode B, is reported beside it as the
    spread between two valid evaluations); the GPU's token must be the
    oracle's argmax wherever the oracle's top-2 margin exceeds the logits'
    observed error."""
    from hybrid_decode_amd import binding as B
    w, st = stack8k
    cfg, kinds = w["cfg"], w["kinds"]
    steps = 16
    snap = _snapshot(st)
    say("capturing the benchmark's step (no logits) into a HIP graph")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step(write_logits=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _restore(st, snap)
    with torch.cuda.graph(graph):
        st.step(write_logits=False)
    torch.cuda.synchronize()
    _restore(st, snap)
    for i in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    g_tokens = st.history.cpu().numpy()[:steps].copy()
    say(f"graph tokens {g_tokens.tolist()}")
    assert np.all(g_tokens >= 0)
    del graph
    _restore(st, snap)

    say("the same tokens layer by layer with logits kept")
    s = rt.stream_ptr()
    ins, outs, logits, tokens = [], [], [], []
    for t in range(steps):
        x = st.x_embed.data_ptr()
        last = st.x_embed
        li_in, li_out = [], []
        for li, kind in enumerate(kinds):
            li_in.append(rt.act_to_host(last, cfg).copy())
            if kind == "gdn":
                B.q35_forward_linear_attention(st.k, st.c, st.layers[li].struct, st.states[li].struct,
                                               st.gdn_scratch.struct, x, st.x_main.data_ptr(), s)
                last = st.x_main
            else:
                B.q35_forward_full_attention_devpos(st.k, st.c, st.layers[li].struct,
                                                    st.full_scratch.struct, st.kvs[li].struct,
                                                    st.inv_freq.data_ptr(), st.positions.data_ptr(),
                                                    x, s)
                last = st.full_scratch.t["x_out"]
            x = last.data_ptr()
            li_out.append(rt.act_to_host(last, cfg).copy())
        B.q35_lm_head_argmax(st.k, st.c, st.final_norm.data_ptr(), st.lm_head.struct, x,
                             st.logits.data_ptr(), st.lm_ws.data_ptr(), st.lm_ws.numel(),
                             st.tokens.data_ptr(), st.positions.data_ptr(), st.history.data_ptr(),
                             st.history_len, st.history_base, st.embed.data_ptr(),
                             st.x_embed.data_ptr(), s)
        torch.cuda.synchronize()
        ins.append(li_in)
        outs.append(li_out)
        logits.append(st.logits.cpu().numpy().copy())
        tokens.append(int(st.tokens.cpu()[0]))
    _restore(st, snap)
    assert tokens == g_tokens.tolist()
    for t in range(steps):
        assert tokens[t] == int(np.argmax(logits[t]))

    say("oracle weights (fp32, dequantised once)")
    olayers, olm = _oracle_weights(w)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    # (b) per-layer teacher forcing: oracle states advanced by the oracle's own layer calls
    lf_states, lf_kvs = list(w["states"]), list(w["kvs"])
    # (a) token teacher forcing: the oracle's own residual stream from the GPU's tokens
    tf_states, tf_kvs = list(w["states"]), list(w["kvs"])
    mb_states, mb_kvs = list(w["states"]), list(w["kvs"])   # the same in Mode B
    prev = w["start_token"]
    worst_b = 0.0
    worst_l = worst_e = worst_g = 0.0
    agree = 0
    for t in range(steps):
        pos = w["ctx"] + t
        for li, kind in enumerate(kinds):
            if kind == "gdn":
                ox, lf_states[li], _ = O.forward_linear_attention(cfg, olayers[li], lf_states[li],
                                                                  ins[t][li])
            else:
                ox, lf_kvs[li], _ = O.forward_full_attention(cfg, olayers[li], lf_kvs[li], inv_h,
                                                             ins[t][li], pos)
            r, e = check(O.act_to_f64(outs[t][li], "bf16"), ox, TOL_BF16, ELEM_BF16, 8, (t, li))
            worst_l, worst_e = max(worst_l, r), max(worst_e, e)
        # the lm_head on the GPU's last layer output
        ol = O.lm_head_logits(cfg, w["final_norm"], olm, O.act_to_f64(outs[t][-1], "bf16"))
        r_lm = rel(logits[t], ol)
        assert r_lm < TOL_GEMV_F16, (t, r_lm)
        # the oracle's own stack from the GPU's previous token
        _, xo, tf_states, tf_kvs = O.decode_stack_step(cfg, kinds, olayers, tf_states, tf_kvs, inv_h,
                                                       w["embed"][prev], pos)
        ol2 = O.lm_head_logits(cfg, w["final_norm"], olm, O.act_to_f64(xo, "bf16"))
        xb = w["embed"][prev]
        for li, kind in enumerate(kinds):
            if kind == "gdn":
                yb, mb_states[li], _ = O.forward_linear_attention(cfg, olayers[li], mb_states[li], xb,
                                                                  mode="B")
            else:
                yb, mb_kvs[li], _ = O.forward_full_attention(cfg, olayers[li], mb_kvs[li], inv_h, xb,
                                                             pos, mode="B")
            xb = O.f64_to_act(yb, "bf16")
        olb = O.lm_head_logits(cfg, w["final_norm"], olm, O.act_to_f64(xb, "bf16"))
        r_tf = rel(logits[t], ol2)
        r_b = rel(olb, ol2)
        worst_g, worst_b = max(worst_g, r_tf), max(worst_b, r_b)
        assert r_tf < TOL_STACK, (t, r_tf)
        err = float(np.max(np.abs(logits[t] - ol2)))
        top2 = np.sort(ol2)[-2:]
        ot = O.greedy(ol2)
        if top2[1] - top2[0] > 2 * err:
            assert ot == tokens[t], (t, ot, tokens[t])
        agree += int(ot == tokens[t])
        say(f"token {t}: {tokens[t]} (oracle {ot}, Mode B {O.greedy(olb)}); lm_head rel {r_lm:.1e}, "
            f"stack logits rel {r_tf:.2e} (Mode B vs A {r_b:.2e})")
        prev = tokens[t]
    say(f"16 tokens: worst layer rel {worst_l:.2e}, element error {worst_e:.3f} RMS, "
        f"stack logits rel {worst_g:.2e} (Mode B vs A up to {worst_b:.2e}); "
        f"oracle argmax agrees on {agree}/{steps}")


def test_stack_4b_ctx65536_sampled_layers_logits_and_token(rt):
    """Config 5: the same stack with every KV cache filled to 65536 positions
    (2.15 GB of bf16 KV), which stresses split-K attention at its longest."""
    w, st = _make_stack(rt, 65536)
    try:
        _check_one_token(rt, w, st, sample_layers=(0, 3, 31))
    finally:
        del st
        torch.cuda.empty_cache()


# --------------------------------------------------------------------------- persistent kernel


@pytest.fixture(scope="module")
def persist8k(rt, stack8k):
    """The same workload run by the persistent decode kernel (an alternative to the
per-layer kernels that the benchmark replays)."""
    w, _ = stack8k
    say("persistent plan over the 8192-context stack")
    return _stack_from(rt, w, persistent=True)


def _check_persistent_token(rt, w, st, sample_layers):
    """One persistent step; every layer's input and output stay in the plan's
    buffers, so each sampled layer is checked against the oracle fed with the
    GPU's own input to it, then sampled logits, the token and the bookkeeping."""
    cfg, kinds = w["cfg"], w["kinds"]
    plan = st.plan
    snap = _snapshot(st)
    x0 = rt.act_to_host(plan.layer_input(0), cfg).copy()
    assert np.array_equal(x0, w["embed"][w["start_token"]])
    say("one persistent decode step")
    st.step()
    torch.cuda.synchronize()
    assert plan.check() == 0
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    pos = w["ctx"]
    for li in sample_layers:
        xin = x0 if li == 0 else rt.act_to_host(plan.layer_input(li), cfg).copy()
        xout = rt.act_to_host(plan.layer_input(li + 1), cfg).copy()
        say(f"oracle check of layer {li} ({kinds[li]})")
        if kinds[li] == "gdn":
            ox, _, _ = O.forward_linear_attention(cfg, w["layers"][li], w["states"][li], xin)
        else:
            ox, _, _ = O.forward_full_attention(cfg, w["layers"][li], w["kvs"][li], inv_h, xin, pos)
        r, e = check(O.act_to_f64(xout, "bf16"), ox, TOL_BF16, ELEM_BF16, 8, li)
        say(f"  layer {li}: rel {r:.2e}, element error {e:.3f} RMS")
    x_last = rt.act_to_host(plan.layer_input(len(kinds)), cfg).copy()
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


def test_persistent_stack_4b_ctx8192_sampled_layers_logits_and_token(rt, stack8k, persist8k):
    w, _ = stack8k
    _check_persistent_token(rt, w, persist8k, sample_layers=(0, 3, 13, 15, 30, 31))


def test_persistent_stack_matches_layer_by_layer(rt, stack8k, persist8k):
    """One token through both paths from the same state, every layer compared.
    GDN layers use the same row arithmetic, so they agree bit for bit until the
    first full-attention layer, whose split-K chunking differs; from there the
    paths differ by fp32 summation order carried through bf16 residuals (the
    greedy tokens may then legitimately differ), within the bf16 tolerance."""
    from hybrid_decode_amd import binding as B
    w, st = stack8k
    ps = persist8k
    cfg, kinds = w["cfg"], w["kinds"]
    sa, sb = _snapshot(st), _snapshot(ps)
    s = rt.stream_ptr()
    x = st.x_embed.data_ptr()
    outs = []
    for li, kind in enumerate(kinds):
        if kind == "gdn":
            B.q35_forward_linear_attention(st.k, st.c, st.layers[li].struct, st.states[li].struct,
                                           st.gdn_scratch.struct, x, st.x_main.data_ptr(), s)
            last = st.x_main
        else:
            B.q35_forward_full_attention_devpos(st.k, st.c, st.layers[li].struct,
                                                st.full_scratch.struct, st.kvs[li].struct,
                                                st.inv_freq.data_ptr(), st.positions.data_ptr(), x, s)
            last = st.full_scratch.t["x_out"]
        x = last.data_ptr()
        torch.cuda.synchronize()
        outs.append(rt.act_to_f32(last, cfg).copy())
    say("persistent step")
    ps.step()
    torch.cuda.synchronize()
    assert ps.plan.check() == 0
    first_full = kinds.index("full")
    worst = 0.0
    for li in range(len(kinds)):
        r = rel(rt.act_to_f32(ps.plan.layer_input(li + 1), cfg), outs[li])
        worst = max(worst, r)
        if li < first_full:
            assert r == 0.0, li
        assert r < TOL_BF16, (li, r)
    say(f"first full layer rel {rel(rt.act_to_f32(ps.plan.layer_input(first_full + 1), cfg), outs[first_full]):.2e}; "
        f"worst layer rel {worst:.2e}")
    assert rel(rt.act_to_f32(ps.plan.layer_input(first_full + 1), cfg), outs[first_full]) < 1e-3
    _restore(st, sa)
    _restore(ps, sb)


def test_persistent_graph_replay_matches_eager(rt, persist8k):
    st = persist8k
    snap = _snapshot(st)
    steps = 4
    say("eager persistent decode of 4 tokens")
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    eager_hist = st.history.cpu().numpy()[:steps].copy()
    eager_logits = st.logits.cpu().numpy().copy()
    eager_state = st.states[0].gdn_state.cpu().numpy().copy()
    eager_k = st.kvs[3].k.cpu().numpy().copy()
    _restore(st, snap)
    say("capturing one persistent step into a HIP graph")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.step()
    torch.cuda.synchronize()
    _restore(st, snap)
    for i in range(steps):
        say(f"persistent graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
    assert st.plan.check() == 0
    assert np.array_equal(st.history.cpu().numpy()[:steps], eager_hist)
    assert np.array_equal(st.logits.cpu().numpy(), eager_logits)
    assert np.array_equal(st.states[0].gdn_state.cpu().numpy(), eager_state)
    assert np.array_equal(st.kvs[3].k.cpu().numpy(), eager_k)
    _restore(st, snap)


def test_persistent_stack_4b_ctx65536_sampled_layers_logits_and_token(rt):
    """Config 5 through the persistent kernel (2.15 GB of bf16 KV)."""
    w, st = _make_stack(rt, 65536, persistent=True)
    try:
        _check_persistent_token(rt, w, st, sample_layers=(0, 3, 31))
    finally:
        del st
        torch.cuda.empty_cache()
