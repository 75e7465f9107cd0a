#!/usr/bin/env python3
"""Batch-1 greedy decode through the Qwen3.5-4B-shaped int8 hybrid stack on one MI355X.

One step = one token through the whole path: 32 layers (24 GDN, 8 gated full
attention over a bf16 KV cache at ~8192 tokens), final RMSNorm, int8 lm_head over
248 320 tokens, greedy argmax and the next token's embedding, all on the device
from one replayed HIP graph.  Prints one JSON line (rank 0).

    python bench.py [--gpus 1] [--steps 128] [--warmup 8] [--ctx 8192] [--kv FORMAT]
                    [--prefill-tokens 4096]

The line also carries "prefill": a prompt of --prefill-tokens
tokens through the same stack with the multi-token prefill calls (timed after
the decode, it overwrites the first cache rows), and the rate of its
dequantising GEMM against the f16 matrix-core peak.  "long_ctx" is decode at a
long context (--long-ctx, default 65536 positions of KV in every full layer,
--long-steps tokens) with the attention steps' own roofline.  "cpu_baseline"
times whole tokens of the oracle on the host, weights dequantised once first.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "batch-1 decode tok/s + achieved HBM GB/s, Qwen3.5-4B-shaped int8 layers"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stack_bytes_per_token(cfg, st, kinds, seq_len: int, kv_bytes: float = 2.0) -> int:
    """Algorithmic HBM bytes of one token at attention length seq_len: every weight
    byte (codes, scales, biases) once, GDN and conv state read + write, conv
    weights, KV rows [0, seq_len) read plus one row appended per full layer
    (kv_bytes per element: 2 for bf16, 1 + 2/16 for Turbo8), the lm_head, the
    embedding row, norm weights and the residual stream."""
    b = st.weight_bytes
    H = cfg.hidden
    for li, kind in enumerate(kinds):
        b += 2 * H * 2 * 2                                   # input_ln + post_ln, residual in/out
        if kind == "gdn":
            b += 2 * cfg.num_v_heads_lin * cfg.k_head_dim_lin * cfg.v_head_dim_lin * 4
            b += 2 * cfg.qkv_total_lin * cfg.conv_kernel_size * 4
            b += cfg.qkv_total_lin * cfg.conv_kernel_size * 2
        else:
            b += int(seq_len * cfg.kv_dim * 2 * kv_bytes)        # K and V rows read
            b += int(cfg.kv_dim * 2 * kv_bytes)                  # append
    b += H * 2 * 2                                           # final norm + embedding row
    return b


def gate_up_bytes(cfg) -> int:
    """Bytes one gate/up launch must move: both matrices (codes + bf16 scales and
    biases), the fp32 residual and norm weight in, the fp32 product out."""
    w = 2 * cfg.intermediate * cfg.hidden * (1 + 4 / 64)
    return int(w + cfg.hidden * (4 + 2) + cfg.intermediate * 4)


# HBM traffic of the dominant kernel from rocprofv3 PMC runs (FETCH_SIZE and
# WRITE_SIZE, calibrated on a device copy of known size), valid only for the
# kernel source it was measured on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemv_traffic.json")
KERNEL_SOURCES = ["hybrid_decode_amd/csrc/gemv_core.h", "hybrid_decode_amd/csrc/gemv_mlp.hip",
                  "hybrid_decode_amd/csrc/gemv.hip", "hybrid_decode_amd/csrc/q35_device.h",
                  "hybrid_decode_amd/csrc/q35_internal.h"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Bytes per launch from the committed PMC summary, or None when it is absent
    or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def copy_bandwidth(torch, nbytes=1 << 29, reps=10):
    """Device-to-device copy rate (read + write bytes per second) for reference."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    return 2 * nbytes / s / 1e9, nbytes


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_weights(w):
    """Every quantised matrix of the stack as dense fp32, dequantised once
    (the oracle's fp32 evaluation of stack-sized GEMVs); returns (layers, lm_head)."""
    import numpy as np

    import oracle as O
    ql = lambda l: {k: (O.QuantMatrix(v, np.float32) if isinstance(v, dict) and "codes" in v else v)
                    for k, v in l.items()}
    layers = [ql(l) for l in w["layers"]]
    for l in layers:
        for v in l.values():
            if isinstance(v, O.QuantMatrix):
                v.dense()
    lm = O.QuantMatrix(w["lm_head"], np.float32)
    lm.dense()
    return layers, lm


def oracle_token(cfg, w, layers, lm, states, kvs, token, pos, kv="bf16"):
    """One whole token of the oracle: the layer loop, final norm, lm_head, greedy."""
    import oracle as O
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    x = w["embed"][token]
    for li, kind in enumerate(w["kinds"]):
        if kind == "gdn":
            y, states[li], _ = O.forward_linear_attention(cfg, layers[li], states[li], x)
        elif kv == "bf16":
            y, kvs[li], _ = O.forward_full_attention(cfg, layers[li], kvs[li], inv, x, pos)
        elif kv == "turbo8":
            from oracle import turbo8 as T8
            y, kvs[li], _ = T8.forward_full_attention_turbo8(cfg, layers[li], kvs[li], inv, x, pos)
        else:
            from oracle import turbo_lm as TL
            y, kvs[li], _ = TL.forward_full_attention(kv, cfg, layers[li], kvs[li], inv, x, pos)
        x = O.f64_to_act(y, cfg.act_dtype)
    return O.greedy(O.lm_head_logits(cfg, w["final_norm"], lm, O.act_to_f64(x, cfg.act_dtype)))


def cpu_baseline(cfg, w, tokens, kv="bf16", n=3):
    """The oracle as it stands, on whole tokens: dense fp32 weights cached once
    (setup not timed), then n tokens at cache positions ctx, ctx + 1, ..., each
    fed the token the GPU chose (teacher forcing); returns the baseline record
    and the cached weights."""
    t0 = time.perf_counter()
    layers, lm = oracle_weights(w)
    setup = time.perf_counter() - t0
    states = list(w["states"])
    kvs = [None if c is None else {k: v for k, v in c.items() if k not in ("capacity", "kv_dtype")}
           for c in w["kvs"]]
    t0 = time.perf_counter()
    for i in range(n):
        oracle_token(cfg, w, layers, lm, states, kvs, tokens[i], w["ctx"] + i, kv)
    t_tok = (time.perf_counter() - t0) / n
    rec = {"value": 1.0 / t_tok, "unit": "tok/s", "cores": blas_threads(), "kind": "oracle",
           "sample": (f"{n} whole tokens of the oracle as it stands ({len(w['kinds'])} layers, final "
                      f"norm, lm_head over {cfg.vocab}, greedy) at cache positions {w['ctx']}.."
                      f"{w['ctx'] + n - 1} ({kv} KV), each fed the token the GPU chose; weights "
                      f"dequantised once to fp32 ({setup:.0f} s, not timed), GEMVs in fp32 BLAS, "
                      f"the rest float64: {t_tok:.2f} s per token"),
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    return rec, (layers, lm)


def graph_kernel_nodes(graph):
    """Kernel nodes of a captured graph (hipGraphGetNodes / hipGraphNodeGetType),
    or None when the runtime cannot be queried."""
    import ctypes as C
    try:
        import torch
        try:
            hip = C.CDLL("libamdhip64.so")
        except OSError:
            hip = C.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        h = C.c_void_p(graph.raw_cuda_graph())
        n = C.c_size_t(0)
        if hip.hipGraphGetNodes(h, None, C.byref(n)) != 0:
            return None
        nodes = (C.c_void_p * n.value)()
        if hip.hipGraphGetNodes(h, nodes, C.byref(n)) != 0:
            return None
        count = 0
        for nd in nodes:
            t = C.c_int(-1)
            if hip.hipGraphNodeGetType(C.c_void_p(nd), C.byref(t)) != 0:
                return None
            count += int(t.value == 0)  # hipGraphNodeTypeKernel
        return count
    except Exception:  # pragma: no cover
        return None


PEAK_MFMA_F16_TFLOPS = 2500.0


def prefill_stack(torch, B, rt, st, kinds, cfg, T, reps=3):
    """T prompt tokens through every layer of the stack (the multi-token prefill
    calls; full layers at cache positions [0, T)); returns ms per pass."""
    import numpy as np
    ws_bytes = B.q35_prefill_workspace_bytes(st.c, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    g = np.random.default_rng(7)
    x0 = torch.from_numpy((g.standard_normal((T, cfg.hidden), dtype=np.float32)).astype(np.float32))
    xa = x0.to("cuda").to(torch.bfloat16).view(torch.int16).contiguous()
    xb = torch.empty_like(xa)
    s = rt.stream_ptr()

    def one_pass():
        x, y = xa, xb
        for li, kind in enumerate(kinds):
            if kind == "gdn":
                B.q35_prefill_linear_attention(st.k, st.c, st.layers[li].struct, st.states[li].struct,
                                               x.data_ptr(), T, y.data_ptr(), ws.data_ptr(), ws_bytes, s)
            else:
                B.q35_prefill_full_attention(st.k, st.c, st.layers[li].struct, st.kvs[li].struct,
                                             st.inv_freq.data_ptr(), x.data_ptr(), T, 0, y.data_ptr(),
                                             ws.data_ptr(), ws_bytes, s)
            x, y = y, x

    one_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        one_pass()
    e1.record()
    torch.cuda.synchronize()
    del ws
    return e0.elapsed_time(e1) / reps


def prefill_gemm_rate(torch, B, rt, st, cfg, T, rounds=2):
    """The prefill's dequantising GEMM at the gate_proj shape (T x intermediate x
    hidden), every layer's weights in turn, each launch dequantising its W to f16
    first (the prefill's own path at this many rows), on seeded N(0, 1) f16 rows (the
    matrix cores draw less power on zero operands and then clock higher, so
    zero rows would overstate the rate); returns (us per launch, flops per launch)."""
    import numpy as np
    g = np.random.default_rng(11)
    x = torch.from_numpy(g.standard_normal((T, cfg.hidden), dtype=np.float32).astype(np.float16)
                         .view(np.int16)).to("cuda")
    y = torch.empty((T, cfg.intermediate), dtype=torch.float32, device="cuda")
    # room for the split area and for W as f16 (dequantised once per launch, timed with it)
    wn = B.PREFILL_GEMM_WORKSPACE_BYTES + 2 * cfg.intermediate * cfg.hidden
    ws = torch.empty(wn, dtype=torch.uint8, device="cuda")
    wp = ws.data_ptr()
    s = rt.stream_ptr()
    B.q35_prefill_gemm(st.k, st.layers[0].q["gate_proj"].struct, x.data_ptr(), T, y.data_ptr(), wp, wn, s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        for L in st.layers:
            B.q35_prefill_gemm(st.k, L.q["gate_proj"].struct, x.data_ptr(), T, y.data_ptr(), wp, wn, s)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (rounds * len(st.layers))
    return us, 2.0 * T * cfg.intermediate * cfg.hidden


def library_gemm_rate(torch, M, N, K, reps=20):
    """For reference: the ROCm BLAS f16 GEMM (torch.mm) on dense f16 operands of
    the same shape, [M, K] x [K, N] with fp32 accumulation inside the library;
    returns TFLOP/s.  Not part of the path (its weights would be twice the bytes
    of the int8 codes); it places the dequantising GEMM against the vendor's."""
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((M, K), dtype=torch.float16, device="cuda", generator=g)
    wt = torch.randn((K, N), dtype=torch.float16, device="cuda", generator=g)
    for _ in range(3):
        torch.mm(x, wt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(x, wt)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del x, wt
    return 2.0 * M * N * K / (us * 1e-6) / 1e12


def prefill_cpu_baseline(cfg, w, layers, n=8):
    """The prefill oracle (the decode step looped over the tokens) on n tokens
    through one GDN and one full-attention layer (dense fp32 weights cached
    beforehand), composed over the stack."""
    import numpy as np

    import oracle as O
    kinds = w["kinds"]
    gi, fi = kinds.index("gdn"), kinds.index("full")
    x = w["embed"][np.arange(n) + 1]
    inv = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    kv = {"k": np.zeros((n, cfg.num_kv_heads, cfg.head_dim), np.uint16),
          "v": np.zeros((n, cfg.num_kv_heads, cfg.head_dim), np.uint16)}
    t0 = time.perf_counter()
    O.prefill.prefill_linear_attention(cfg, layers[gi], w["states"][gi], x)
    t_gdn = (time.perf_counter() - t0) / n
    t0 = time.perf_counter()
    O.prefill.prefill_full_attention(cfg, layers[fi], kv, inv, x, 0)
    t_full = (time.perf_counter() - t0) / n
    t_tok = kinds.count("gdn") * t_gdn + kinds.count("full") * t_full
    return 1.0 / t_tok, (f"prefill oracle as it stands (the decode step looped over the tokens; "
                         f"dense fp32 weights cached, GEMVs in fp32 BLAS, the rest float64) on {n} "
                         f"tokens through one GDN layer ({t_gdn:.3f}s/token) and one full layer at "
                         f"cache positions 0..{n - 1} ({t_full:.3f}s/token), composed over "
                         f"{kinds.count('gdn')} + {kinds.count('full')} layers")


def long_context(torch, B, rt, synth, workloads, args, kv_bytes):
    """Decode at a long context: the same 32-layer stack with every KV cache
    filled to args.long_ctx positions, args.long_steps tokens from one replayed
    graph; plus the attention steps alone (q35_attention_devpos: split, norms,
    RoPE, append, split-K attention, merge and gate) timed on every full
    layer's cache, the kernel the long context stresses."""
    import numpy as np
    ctx, K2, W2 = args.long_ctx, args.long_steps, 4
    log(f"long context: generating the stack with KV at {ctx} positions")
    w = workloads.stack_4b(synth.Gen(0), num_layers=args.layers, ctx=ctx, extra=W2 + K2 + 64, kv=args.kv)
    cfg, kinds = w["cfg"], w["kinds"]
    st = rt.DecodeStack(cfg, kinds, w["layers"], w["states"], w["kvs"], w["embed"], w["final_norm"],
                        w["lm_head"], start_pos=ctx, start_token=w["start_token"],
                        history_len=W2 + K2 + 8)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.step(write_logits=False)
    for _ in range(W2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K2):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    tok_s = K2 / (ms / 1e3)
    L_mid = ctx + W2 + K2 // 2 + 1
    bpt = stack_bytes_per_token(cfg, st, kinds, L_mid, kv_bytes)
    hist = st.history.cpu().numpy()[:W2 + K2]
    assert np.all(hist >= 0) and np.all(hist < cfg.vocab), "decode produced invalid tokens"
    log(f"long context {ctx}: {K2} tokens in {ms:.2f} ms: {ms / K2 * 1e3:.1f} us/token, {tok_s:.1f} tok/s, "
        f"{bpt * tok_s / 1e9:.0f} GB/s")
    # the attention steps alone, every full layer's cache in turn (the append
    # rewrites row positions[0] with the same values each time)
    s = rt.stream_ptr()
    full = [i for i, k in enumerate(kinds) if k == "full"]
    sc = st.full_scratch
    call = lambda li: B.q35_attention_devpos(st.k, st.c, st.layers[li].struct, sc.struct,
                                             st.kvs[li].struct, st.inv_freq.data_ptr(),
                                             st.positions.data_ptr(), s)
    for li in full:
        call(li)
    torch.cuda.synchronize()
    R = 4
    torch.cuda._sleep(100_000_000)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(R):
        for li in full:
            call(li)
    a1.record()
    torch.cuda.synchronize()
    attn_us = a0.elapsed_time(a1) * 1e3 / (R * len(full))
    L = int(st.positions.cpu()[0]) + 1
    attn_bytes = int(L * cfg.kv_dim * 2 * kv_bytes)   # K and V rows read (the append included)
    attn_gbs = attn_bytes / (attn_us * 1e-6) / 1e9
    log(f"long context {ctx}: attention steps {attn_us:.1f} us per layer, {attn_gbs:.0f} GB/s")
    out = {"ctx_start": ctx, "steps": K2, "warmup": W2, "value": round(tok_s, 2), "unit": "tok/s",
           "ms_per_step": round(ms / K2, 4), "bytes_per_token": bpt,
           "hbm_gbs": round(bpt * tok_s / 1e9, 1), "hbm_frac": round(bpt * tok_s / 1e9 / PEAK_HBM_GBS, 4),
           "roofline": {"bound": "hbm",
                        "kernel": "attn_partial_kernel + attn_merge_kernel (q35_attention_devpos)",
                        "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(attn_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "bytes_per_launch": attn_bytes, "us_per_launch": round(attn_us, 2)}}
    del graph, st
    torch.cuda.empty_cache()
    return out


def layer_configs(torch, B, rt, synth, workloads, rounds=5, copies=6):
    """One 4B GDN layer for 256 sequential steps (GDN state N(0, 0.1), conv state
    N(0, 1), a fresh N(0, 1) input row each step) and one 4B full-attention layer
    for 64 steps at cache positions 4096..4159 (bf16 KV rows [0, 4096) N(0, 1)).
    Step t runs on device copy t % copies of the layer's weights: identical
    bytes at distinct addresses, more of them than the 256 MB last-level cache
    holds, so every step streams its weights from HBM (the copies share one
    state or one KV cache, so the results equal one copy's).  All steps of a run
    are one captured HIP graph; per-step time from the median and the fastest of
    `rounds` replays.  The same graph on one copy gives the cache-warm figure
    (its weights fit in the last-level cache), reported beside it."""
    import numpy as np
    s_of = rt.stream_ptr
    out = {}

    def timed(graph, steps):
        graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / steps)
        return float(np.median(ts)), float(min(ts))

    def entry(kind, workload, steps, bpstep, rot, warm):
        (med, mn), (wmed, _) = rot, warm
        gbs = bpstep / (med * 1e-6) / 1e9
        log(f"{kind} layer, {steps} steps over {copies} weight copies: {med:.2f} us/step "
            f"(min {mn:.2f}), {gbs:.0f} GB/s; one copy (cache-warm): {wmed:.2f} us/step")
        return {"workload": workload, "steps": steps, "weight_copies": copies, "rounds": rounds,
                "us_per_step": round(med, 2), "us_per_step_min": round(mn, 2),
                "bytes_per_step": bpstep, "hbm_gbs": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "us_per_step_one_copy_cache_warm": round(wmed, 2)}

    # GDN layer
    w = workloads.gdn_layer_4b(synth.Gen(0))
    cfg, H = w["cfg"], w["cfg"].hidden
    k, c = rt.kernels(0), rt.cfg_struct(cfg)
    Ls = [rt.GdnLayerDev(w["layer"]) for _ in range(copies)]
    S, scr = rt.GdnStateDev(w["state"]), rt.GdnScratchDev(cfg)
    xs = rt.to_dev(np.stack(w["xs"]))
    xbuf = rt.act_empty(cfg, H)
    steps = xs.shape[0]
    graphs = []
    for ncopy in (copies, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(steps):
                B.q35_forward_linear_attention(k, c, Ls[t % ncopy].struct, S.struct, scr.struct,
                                               xs[t].data_ptr(), xbuf.data_ptr(), s_of())
        graphs.append(g)
    rot, warm = timed(graphs[0], steps), timed(graphs[1], steps)
    bpstep = (Ls[0].weight_bytes + 2 * H * 2 * 2
              + 2 * cfg.num_v_heads_lin * cfg.k_head_dim_lin * cfg.v_head_dim_lin * 4
              + 2 * cfg.qkv_total_lin * cfg.conv_kernel_size * 4 + cfg.qkv_total_lin * cfg.conv_kernel_size * 2)
    assert torch.isfinite(S.gdn_state).all(), "GDN state not finite"
    out["gdn"] = entry("GDN", f"one Qwen3.5-4B-shaped GDN layer (int8 g64 weights, bf16 activations), "
                              f"{steps} sequential single-token steps", steps, bpstep, rot, warm)
    del graphs, Ls, S, scr, xs
    torch.cuda.empty_cache()

    # full-attention layer
    w = workloads.full_layer_4b(synth.Gen(0))
    cfg, start = w["cfg"], w["start"]
    c = rt.cfg_struct(cfg)
    Ls = [rt.FullLayerDev(w["layer"]) for _ in range(copies)]
    kv = rt.KvCacheDev(w["kv"])
    fs = rt.FullScratchDev(cfg, kv.capacity)
    inv = rt.inv_freq_dev(cfg)
    xs = rt.to_dev(np.stack(w["xs"]))
    steps = xs.shape[0]
    pos = torch.arange(start, start + steps, dtype=torch.int32, device="cuda")
    graphs = []
    for ncopy in (copies, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(steps):
                B.q35_forward_full_attention(k, c, Ls[t % ncopy].struct, fs.struct, kv.struct,
                                             inv.data_ptr(), pos[t:t + 1].data_ptr(), xs[t].data_ptr(),
                                             start + t, start + t + 1, s_of())
        graphs.append(g)
    rot, warm = timed(graphs[0], steps), timed(graphs[1], steps)
    mean_len = start + (steps + 1) / 2.0   # rows attended per step, on average
    bpstep = int(Ls[0].weight_bytes + 2 * H * 2 * 2 + mean_len * cfg.kv_dim * 2 * 2 + cfg.kv_dim * 2 * 2)
    out["full"] = entry("full-attention", f"one Qwen3.5-4B-shaped gated full-attention layer (int8 g64 "
                                          f"weights, bf16 activations, bf16 KV rows [0, {start}) N(0, 1)), "
                                          f"{steps} steps at cache positions {start}..{start + steps - 1}",
                        steps, bpstep, rot, warm)
    del graphs, Ls, kv, fs, xs
    torch.cuda.empty_cache()
    return out


KV_FORMATS = ["bf16", "turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]


def attention_formats(torch, B, rt, synth, pos, rounds=8, copies=8):
    """The attention steps alone (q35_attention_devpos) at cache position pos for
    every KV format: `copies` device copies of one layer's synthetic cache (more
    bytes than the last-level cache holds), each quantised format with the
    sparse-V gate at the pages' default and off.  Host-event time per layer."""
    from synth import qwen3_5_4b, full_layer, kv_cache, kv_cache_turbo8, kv_cache_lm
    cfg = qwen3_5_4b("bf16")
    g = synth.Gen(0)
    cap = pos + 64
    layer = rt.FullLayerDev(full_layer(g, cfg, "af.L"))
    inv = rt.inv_freq_dev(cfg)
    posd = torch.tensor([pos], dtype=torch.int32, device="cuda")
    out = {"workload": f"attention steps of one Qwen3.5-4B full-attention layer at cache position {pos}, "
                       f"{copies} cache copies in turn", "pos": pos, "formats": {}}
    for fmt in KV_FORMATS:
        log(f"attention at {pos}: {fmt}")
        if fmt == "bf16":
            kv = kv_cache(g, cfg, f"af.{fmt}", cap, pos)
        elif fmt == "turbo8":
            kv = kv_cache_turbo8(g, cfg, f"af.{fmt}", cap, pos)
        else:
            kv = kv_cache_lm(g, cfg, f"af.{fmt}", cap, pos, fmt)
        res = {}
        for tau in ([None] if fmt == "bf16" else [rt.KvCacheDev.SPARSE_V_DEFAULT, 0.0]):
            kvs = [rt.KvCacheDev(kv) if tau is None else rt.KvCacheDev(kv, sparse_v=tau) for _ in range(copies)]
            scr = rt.FullScratchDev(cfg, cap)
            scr.t["q_full"].normal_()
            scr.t["k"].normal_()
            scr.t["v"].normal_()
            s = rt.stream_ptr()

            def run():
                for kvd in kvs:
                    B.q35_attention_devpos(rt.kernels(0), rt.cfg_struct(cfg), layer.struct, scr.struct,
                                           kvd.struct, inv.data_ptr(), posd.data_ptr(), s)
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(50_000_000)
            e0.record()
            for _ in range(rounds):
                run()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (rounds * copies)
            res["default" if tau else ("off" if tau == 0.0 else "exact")] = round(us, 2)
            del kvs, scr
            torch.cuda.empty_cache()
        out["formats"][fmt] = res
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dominant-rounds", type=int, default=4)
    ap.add_argument("--prefill-tokens", type=int, default=4096,
                    help="also time a prompt of this many tokens through the stack (0: skip)")
    ap.add_argument("--long-ctx", type=int, default=65536,
                    help="also time decode with every KV cache filled to this many positions (0: skip)")
    ap.add_argument("--long-steps", type=int, default=32)
    ap.add_argument("--no-layer-configs", action="store_true",
                    help="skip the single-layer runs (GDN 256 steps, full attention 64 steps, rotated weights)")
    ap.add_argument("--path", choices=["layers", "xcd"], default="layers",
                    help="decode launches: per-layer kernels, or the XCD-split plan (q35_xcd_*)")
    ap.add_argument("--attn-formats", type=int, default=0, metavar="POS",
                    help="only time the attention steps at cache position POS for every KV format "
                         "(sparse-V gate at its default and off) and print one JSON line")
    ap.add_argument("--kv", choices=["bf16", "turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v",
                                     "bf16k_turbo3v", "bf16k_turbo2v"], default="bf16",
                    help="KV cache format of the full-attention layers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path here is single-device "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from synth import workloads
    from hybrid_decode_amd import build as hb
    if not hb.is_built():
        hb.build()
    from hybrid_decode_amd import binding as B
    from hybrid_decode_amd import runtime as rt

    torch.cuda.set_device(0)
    rt.kernels(0)
    if args.attn_formats > 0:
        print(json.dumps(attention_formats(torch, B, rt, synth, args.attn_formats)), flush=True)
        return
    K, W = args.steps, args.warmup
    t0 = time.time()
    gen = synth.Gen(0)
    log(f"generating the {args.layers}-layer stack (ctx {args.ctx})")
    w = workloads.stack_4b(gen, num_layers=args.layers, ctx=args.ctx, extra=W + K + 64,
                           progress=lambda i: log(f"  layer {i} generated") if i % 8 == 7 else None,
                           kv=args.kv)
    # bytes per K and V element, averaged over the two
    lm_bits = {"turbo4": 4, "turbo3": 3, "turbo2": 2, "bf16k_turbo4v": 4, "bf16k_turbo3v": 3,
               "bf16k_turbo2v": 2}
    if args.kv in lm_bits:
        side = lm_bits[args.kv] / 8 + 1.0 / 16
        kv_bytes = (side + (2.0 if args.kv.startswith("bf16k") else side)) / 2
    else:
        kv_bytes = {"bf16": 2.0, "turbo8": 1.0 + 2.0 / 16}[args.kv]
    cfg, kinds = w["cfg"], w["kinds"]
    log(f"generated in {time.time() - t0:.1f}s; uploading")
    st = rt.DecodeStack(cfg, kinds, w["layers"], w["states"], w["kvs"], w["embed"],
                        w["final_norm"], w["lm_head"], start_pos=args.ctx,
                        start_token=w["start_token"], history_len=W + K + 8, xcd=args.path == "xcd")
    torch.cuda.synchronize()
    log(f"resident weights {st.weight_bytes / 1e9:.3f} GB; decode path: {args.path}")

    # one decode token captured once, replayed every step
    graph = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(graph):
        st.step(write_logits=False)
    launches = graph_kernel_nodes(graph)
    graph.instantiate()
    log(f"graph captured: {launches} kernel launches per token")
    for _ in range(W):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / K
    tok_s = K / (ms / 1e3)
    L_mid = args.ctx + W + K // 2 + 1
    bpt = stack_bytes_per_token(cfg, st, kinds, L_mid, kv_bytes)
    hist = st.history.cpu().numpy()[:W + K]
    assert np.all(hist >= 0) and np.all(hist < cfg.vocab), "decode produced invalid tokens"
    if st.plan is not None:
        err = st.plan.check()
        assert err == 0, f"the decode plan reported error word {err:#x}"
    log(f"{K} tokens in {ms:.2f} ms: {ms_per_step * 1e3:.1f} us/token, {tok_s:.1f} tok/s, "
        f"{bpt * tok_s / 1e9:.0f} GB/s")

    # per-layer device time for one eager token (launches queued behind a spin so
    # the host never starves the device)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(kinds) + 2)]
    torch.cuda._sleep(200_000_000)
    s = rt.stream_ptr()
    x = st.x_embed.data_ptr()
    evs[0].record()
    for li, kind in enumerate(kinds):
        if kind == "gdn":
            x = B.q35_forward_linear_attention(st.k, st.c, st.layers[li].struct, st.states[li].struct,
                                               st.gdn_scratch.struct, x, st.x_main.data_ptr(), s)
        else:
            x = B.q35_forward_full_attention_devpos(st.k, st.c, st.layers[li].struct,
                                                    st.full_scratch.struct, st.kvs[li].struct,
                                                    st.inv_freq.data_ptr(), st.positions.data_ptr(), x, s)
        evs[li + 1].record()
    B.q35_lm_head_argmax(st.k, st.c, st.final_norm.data_ptr(), st.lm_head.struct, x, None,
                         st.lm_ws.data_ptr(), st.lm_ws.numel(), st.tokens.data_ptr(),
                         st.positions.data_ptr(), None, 0, 0, st.embed.data_ptr(),
                         st.x_embed.data_ptr(), s)
    evs[-1].record()
    torch.cuda.synchronize()
    lay = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(len(kinds))]
    gdn_us = float(np.mean([t for t, k in zip(lay, kinds) if k == "gdn"]))
    full_us = float(np.mean([t for t, k in zip(lay, kinds) if k == "full"]))
    lm_us = evs[-2].elapsed_time(evs[-1]) * 1e3
    log(f"eager token: GDN layer {gdn_us:.1f} us, full layer {full_us:.1f} us, lm_head {lm_us:.1f} us")

    # dominant kernel: the post-norm + gate/up SwiGLU GEMV, every layer's weights in
    # turn (distinct addresses: nothing is served from the 256 MB last-level cache)
    x_resid = torch.randn(cfg.hidden, dtype=torch.float32, device="cuda")
    mlp = torch.empty(cfg.intermediate, dtype=torch.float32, device="cuda")
    layers = st.layers
    R = args.dominant_rounds
    torch.cuda._sleep(100_000_000)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(R):
        for L in layers:
            B.q35_gate_up_swiglu(st.k, st.c, L.t["post_ln"].data_ptr(), L.q["gate_proj"].struct,
                                 L.q["up_proj"].struct, x_resid.data_ptr(), mlp.data_ptr(), s)
    d1.record()
    torch.cuda.synchronize()
    dom_us = d0.elapsed_time(d1) * 1e3 / (R * len(layers))
    dom_bytes = gate_up_bytes(cfg)
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    log(f"gate/up GEMV: {dom_us:.2f} us/launch, {dom_gbs:.0f} GB/s")
    copy_gbs, copy_bytes = copy_bandwidth(torch)
    log(f"device copy of {copy_bytes >> 20} MiB: {copy_gbs:.0f} GB/s (read + write)")
    traffic = measured_traffic()

    gpu_tokens = [int(t) for t in hist[:4]]
    first_token = w["start_token"]

    prefill = None
    if args.prefill_tokens > 0:
        T = min(args.prefill_tokens, min(kv.capacity for kv in st.kvs if kv is not None))
        pf_ms = prefill_stack(torch, B, rt, st, kinds, cfg, T)
        g_us, g_flops = prefill_gemm_rate(torch, B, rt, st, cfg, T)
        g_tf = g_flops / (g_us * 1e-6) / 1e12
        lib_tf = library_gemm_rate(torch, T, cfg.intermediate, cfg.hidden)
        log(f"library f16 GEMM (torch.mm) on the same shape: {lib_tf:.0f} TFLOP/s")
        log(f"prefill of {T} tokens through {len(kinds)} layers: {pf_ms:.2f} ms ({T / pf_ms * 1e3:.0f} tok/s); "
            f"GEMM {T}x{cfg.intermediate}x{cfg.hidden}: {g_us:.1f} us, {g_tf:.0f} TFLOP/s")
        prefill = {
            "tokens": T, "ms": round(pf_ms, 3), "tok_s": round(T / pf_ms * 1e3, 1),
            "workload": (f"{T}-token prompt (synthetic bf16 rows) through the {len(kinds)}-layer stack, "
                         f"full layers at cache positions 0..{T - 1}"
                         + ("" if args.kv == "bf16" else f", {args.kv} KV caches")),
            "roofline": {"bound": "mfma", "kernel": "q35_prefill_gemm: pf::dequant_kernel (W to f16) + "
                                                    "pf::gemm_kernel<0, 256, W16> (f16 GEMM, "
                                                    f"{T} x {cfg.intermediate} x {cfg.hidden}), per call",
                         "achieved": round(g_tf, 1), "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(g_tf / PEAK_MFMA_F16_TFLOPS, 4), "traffic": None,
                         "flops_per_launch": g_flops, "us_per_launch": round(g_us, 2),
                         "library_f16_gemm_tflops": round(lib_tf, 1)},
        }

    kv_desc = {"bf16": "bf16", "turbo8": "Turbo8 (WHT-rotated E4M3 + bf16 scale per 16)"}.get(args.kv)
    if kv_desc is None:
        b = lm_bits[args.kv]
        lm = f"Turbo{b} (WHT-rotated {b}-bit Lloyd-Max + E4M3 scale per 16)"
        kv_desc = f"bf16 K + {lm} V" if args.kv.startswith("bf16k") else f"{lm} K and V"
    result = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"Qwen3.5-4B-shaped {args.layers}-layer hybrid stack "
                         f"({kinds.count('gdn')} GDN + {kinds.count('full')} gated full attention), "
                         f"int8 g64 weights, bf16 activations, {kv_desc} KV cache, int8 lm_head "
                         f"over {cfg.vocab}, greedy decode from cache position {args.ctx}"),
            "layers": args.layers, "ctx_start": args.ctx, "hidden": cfg.hidden,
            "intermediate": cfg.intermediate, "vocab": cfg.vocab, "batch": 1,
            "kv": args.kv,
            "storage": f"u8 codes + bf16 scale/bias per 64, bf16 activations, {kv_desc} KV, fp32 GDN state",
            "arithmetic": ("GEMV products of f16 x (rounded per 16-element chunk) and exact f16 "
                           "codes, fp32 sums; norms, softmax, recurrence and state in fp32"),
            "launch": "one HIP graph per token",
            "launches_per_token": launches,
        },
        "bytes_per_token": bpt,
        "hbm_gbs": round(bpt * tok_s / 1e9, 1),
        "hbm_frac": round(bpt * tok_s / 1e9 / PEAK_HBM_GBS, 4),
        "gdn_layer_us": round(gdn_us, 2),
        "full_layer_us": round(full_us, 2),
        "lm_head_us": round(lm_us, 2),
        "copy_gbs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel<2560,true> (post-norm gate/up SwiGLU)",
                     "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": dom_bytes, "us_per_launch": round(dom_us, 3)},
    }
    if args.long_ctx > 0:
        # the same stack with every KV cache filled to long_ctx positions
        del graph, st
        torch.cuda.empty_cache()
        result["long_ctx"] = long_context(torch, B, rt, synth, workloads, args, kv_bytes)
    if not args.no_layer_configs and args.kv == "bf16":
        result["layer_configs"] = layer_configs(torch, B, rt, synth, workloads)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on whole tokens (weights dequantised once first)")
        toks = [first_token] + gpu_tokens
        result["cpu_baseline"], (olayers, _) = cpu_baseline(cfg, w, toks, args.kv)
        log(f"oracle: {result['cpu_baseline']['value']:.4f} tok/s "
            f"({result['cpu_baseline']['sample'].rsplit(': ', 1)[-1]})")
    if prefill is not None:
        if not args.no_cpu_baseline:
            v, note = prefill_cpu_baseline(cfg, w, olayers)
            prefill["cpu_baseline"] = {"value": v, "unit": "tok/s", "kind": "oracle", "sample": note,
                                       "cores": result["cpu_baseline"]["cores"]}
            log(f"prefill oracle: {v:.4f} tok/s")
        result["prefill"] = prefill
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
