"""GPU parity of the layer loop: the tiny two-layer hybrid at every step, and the
4B-shaped stack (real lm_head, KV at 8192) on sampled layers, the logits and the
greedy token, plus HIP-graph replay against eager execution."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import workloads
from gpu_common import TOL_BF16, TOL_F32, TOL_GEMV_F16, rel, say

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
        assert rel(rt.act_to_f32(fs.t["x_out"], cfg), ox) < TOL_F32, t
    assert rel(S0.to_host()["gdn_state"], states[0]["gdn_state"]) < TOL_F32


@pytest.fixture(scope="module")
def stack8(rt):
    """The 4B stack at 8 layers (two full-attention layers, ctx 8192): the same shapes,
    launches and lm_head as the 32-layer benchmark stack, fewer layers."""
    say("generating the 8-layer 4B stack")
    g = synth.Gen(0)
    w = workloads.stack_4b(g, num_layers=8, ctx=8192, extra=64)
    st = rt.DecodeStack(w["cfg"], w["kinds"], w["layers"], w["states"], w["kvs"], w["embed"],
                        w["final_norm"], w["lm_head"], start_pos=w["ctx"],
                        start_token=w["start_token"], history_len=64)
    torch.cuda.synchronize()
    return w, st


def _snapshot(st):
    return ([None if s is None else (s.conv1d_state.clone(), s.gdn_state.clone()) for s in st.states],
            [None if kv is None else (kv.k.clone(), kv.v.clone()) for kv in st.kvs],
            st.positions.clone(), st.tokens.clone(), st.x_embed.clone())


def _restore(st, snap):
    ss, kk, p, t, x = snap
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
    st.x_embed.copy_(x)
    st.history.fill_(-1)


def test_stack_4b_sampled_layers_logits_and_token(rt, stack8):
    from hybrid_decode_amd import binding as B
    w, st = stack8
    cfg, kinds = w["cfg"], w["kinds"]
    snap = _snapshot(st)
    # embedding of the start token, bit-exact
    assert np.array_equal(rt.act_to_host(st.x_embed, cfg), w["embed"][w["start_token"]])
    # run the layers one by one, keeping every layer's input and output
    s = rt.stream_ptr()
    x = st.x_embed.data_ptr()
    ins, outs = [], []
    for li, kind in enumerate(kinds):
        say(f"4B stack layer {li} ({kind})")
        ins.append(rt.act_to_host(st.x_embed if li == 0 else last, cfg).copy())
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
        outs.append(rt.act_to_host(last, cfg).copy())
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    pos = w["ctx"]
    for li in (0, 1, 3, 7):   # GDN (first), GDN, full attention, full attention (last)
        say(f"oracle check of layer {li}")
        if kinds[li] == "gdn":
            ox, _, _ = O.forward_linear_attention(cfg, w["layers"][li], w["states"][li], ins[li])
        else:
            ox, _, _ = O.forward_full_attention(cfg, w["layers"][li], w["kvs"][li], inv_h, ins[li], pos)
        assert rel(O.act_to_f64(outs[li], "bf16"), ox) < TOL_BF16, li
    # lm_head + greedy token on the last layer's output
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
    h = O.rms_norm(O.act_to_f64(outs[-1], "bf16"), w["final_norm"], cfg.rms_eps)
    ref = O.dequant({k: v[rows] for k, v in w["lm_head"].items()}).astype(np.float64) @ h
    r = rel(g[rows], ref)
    say(f"sampled logits rel {r:.2e}")
    assert r < TOL_GEMV_F16
    assert tok == int(np.argmax(g))
    assert int(st.positions.cpu()[0]) == pos + 1
    _restore(st, snap)


def test_stack_4b_graph_replay_matches_eager(rt, stack8):
    w, st = stack8
    snap = _snapshot(st)
    steps = 6
    say("eager decode of 6 tokens")
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    eager_hist = st.history.cpu().numpy()[:steps].copy()
    eager_logits = st.logits.cpu().numpy().copy()
    eager_state = st.states[0].gdn_state.cpu().numpy().copy()
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
    _restore(st, snap)
