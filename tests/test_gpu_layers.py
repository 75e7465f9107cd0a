"""GPU parity of the two layer forwards against the oracle.

Tiny config (fp32 activations): every step and every dump tap at rel 1e-3.
4B config (bf16 activations): layer outputs at rel 2e-2; the fp32 GDN state
after 64 steps at rel 1e-3; KV-append placement bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import workloads
from gpu_common import ELEM_BF16, ELEM_F32, TOL_BF16, TOL_F32, check, rel, say

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


GDN_TAPS = {  # scratch tap -> oracle tap
    "x_norm": "gdn_x_norm", "qkv": "gdn_qkv_pre", "qkv_smooth": "gdn_qkv_smooth", "y": "gdn_y",
    "y_norm": "gdn_y_norm", "out": "gdn_out", "x_resid": "gdn_x_resid", "z": "z", "gate": "gate",
    "beta": "beta", "dt_raw": "dt_raw", "b_raw": "b_raw", "x_norm2": "x_norm2",
    "gate_act": "gate_act", "up_act": "up_act",
}
FULL_TAPS = {
    "x_norm": "x_norm", "q_full": "q_full", "k": "k", "v": "v", "q_norm_out": "q_norm_out",
    "k_norm_out": "k_norm_out", "attn_out": "attn_out", "gated_attn": "gated_attn", "o": "o",
    "x_resid": "x_resid", "x_norm2": "x_norm2", "gate_act": "gate_act", "up_act": "up_act",
}


def test_gdn_layer_tiny_fp32_every_step_and_tap(rt, gen):
    cfg = synth.tiny("f32")
    layer = synth.gdn_layer(gen, cfg, "gpu.tg")
    st = synth.gdn_state(gen, cfg, "gpu.tg", gdn_std=0.1, conv_std=1.0)
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(st)
    scr = rt.GdnScratchDev(cfg, taps=True)
    x_buf = rt.act_empty(cfg, cfg.hidden)
    ost = st
    for t in range(16):
        say(f"tiny GDN step {t}")
        x = gen.act(f"gpu.tg.x{t}", (cfg.hidden,), "f32")
        xin = rt.to_dev(x)
        rt.forward_linear_attention(cfg, L, S, scr, xin, x_buf)
        torch.cuda.synchronize()
        ox, ost, taps = O.forward_linear_attention(cfg, layer, ost, x)
        check(rt.act_to_f32(x_buf, cfg), ox, TOL_F32, ELEM_F32, 24, t)
        for k, ok in GDN_TAPS.items():
            check(scr.t[k].cpu().numpy(), taps[ok], TOL_F32, ELEM_F32, 24, (t, k))
        assert np.array_equal(rt.act_to_host(scr.t["x_final"], cfg), rt.act_to_host(x_buf, cfg))
        gst = S.to_host()
        assert rel(gst["gdn_state"], ost["gdn_state"]) < TOL_F32, t
        assert rel(gst["conv1d_state"], ost["conv1d_state"]) < 1e-6, t


def test_gdn_layer_output_may_alias_input(rt, gen):
    cfg = synth.tiny("bf16")
    layer = synth.gdn_layer(gen, cfg, "gpu.alias")
    st = synth.gdn_state(gen, cfg, "gpu.alias", gdn_std=0.1, conv_std=1.0)
    x = gen.act("gpu.alias.x", (cfg.hidden,), "bf16")
    L = rt.GdnLayerDev(layer)
    scr = rt.GdnScratchDev(cfg)
    S1, S2 = rt.GdnStateDev(st), rt.GdnStateDev(st)
    a_in, a_out = rt.to_dev(x), rt.act_empty(cfg, cfg.hidden)
    b = rt.to_dev(x)
    say("GDN aliasing: separate buffers")
    rt.forward_linear_attention(cfg, L, S1, scr, a_in, a_out)
    say("GDN aliasing: x_buf == x_in")
    rt.forward_linear_attention(cfg, L, S2, scr, b, b)
    torch.cuda.synchronize()
    assert torch.equal(a_out, b)


def test_gdn_dump_hook_receives_named_taps(rt, gen):
    from hybrid_decode_amd import binding as B
    cfg = synth.tiny("f32")
    layer = synth.gdn_layer(gen, cfg, "gpu.dump")
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(synth.gdn_state(gen, cfg, "gpu.dump"))
    scr = rt.GdnScratchDev(cfg, taps=True)
    x = rt.to_dev(gen.act("gpu.dump.x", (cfg.hidden,), "f32"))
    out = rt.act_empty(cfg, cfg.hidden)
    seen = {}

    def dump(ctx, name, p, n):
        seen[name.decode()] = (p, n)

    say("GDN dump hook")
    rt.forward_linear_attention(cfg, L, S, scr, x, out, dump=dump)
    assert list(seen) == ["gdn_x_norm", "gdn_qkv_pre", "gdn_qkv_smooth", "gdn_y", "gdn_y_norm",
                          "gdn_out", "gdn_x_resid", "gdn_x_final"]
    assert seen["gdn_y"] == (scr.t["y"].data_ptr(), cfg.z_dim_lin)
    assert seen["gdn_qkv_pre"][1] == cfg.qkv_total_lin


def test_full_layer_tiny_fp32_every_step_tap_and_append(rt, gen):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "gpu.tf")
    cap = 16
    kv = synth.kv_cache(gen, cfg, "gpu.tf", cap, 0)
    kv["k"][:] = NAN_BF16        # sentinel: any read of an unwritten row poisons the output
    kv["v"][:] = NAN_BF16
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    scr = rt.FullScratchDev(cfg, cap, taps=True)
    inv = rt.inv_freq_dev(cfg)
    okv = {"k": kv["k"].copy(), "v": kv["v"].copy()}
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    for t in range(cap):
        say(f"tiny full-attention step {t}")
        x = gen.act(f"gpu.tf.x{t}", (cfg.hidden,), "f32")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        before = KVd.to_host()
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), t)
        torch.cuda.synchronize()
        ox, okv, taps = O.forward_full_attention(cfg, layer, okv, inv_h, x, t)
        check(rt.act_to_f32(scr.t["x_out"], cfg), ox, TOL_F32, ELEM_F32, 24, t)
        for k, ok in FULL_TAPS.items():
            check(scr.t[k].cpu().numpy(), taps[ok], TOL_F32, ELEM_F32, 24, (t, k))
        after = KVd.to_host()
        for side in ("k", "v"):
            changed = np.nonzero(np.any(after[side] != before[side], axis=(1, 2)))[0].tolist()
            assert changed == [t], (side, t, changed)
            assert rel(O.bf16_to_f64(after[side][t]), O.bf16_to_f64(okv[side][t])) < 1e-2
        # the stored k row is the bf16 rounding of the post-RoPE k the kernel reports
        kn = scr.t["k_norm_out"].cpu().numpy().reshape(cfg.num_kv_heads, cfg.head_dim)
        assert np.array_equal(after["k"][t], O.f64_to_bf16(kn.astype(np.float64)))
        vv = scr.t["v"].cpu().numpy().reshape(cfg.num_kv_heads, cfg.head_dim)
        assert np.array_equal(after["v"][t], O.f64_to_bf16(vv.astype(np.float64)))


def test_gdn_layer_4b_bf16_256_steps_and_state(rt, gen):
    """Config 2: 256 sequential steps; every output within the bf16 tolerance, the
    fp32 GDN and conv states within 1e-3 after 64 steps (and reported at 256)."""
    w = workloads.gdn_layer_4b(gen, steps=256)
    cfg, layer, st = w["cfg"], w["layer"], w["state"]
    L, S = rt.GdnLayerDev(layer), rt.GdnStateDev(st)
    scr = rt.GdnScratchDev(cfg)
    x_buf = rt.act_empty(cfg, cfg.hidden)
    ost = st
    worst = worst_e = 0.0
    for t, x in enumerate(w["xs"]):
        if t % 32 == 0:
            say(f"4B GDN step {t}")
        rt.forward_linear_attention(cfg, L, S, scr, rt.to_dev(x), x_buf)
        ox, ost, _ = O.forward_linear_attention(cfg, layer, ost, x)
        torch.cuda.synchronize()
        r, e = check(rt.act_to_f32(x_buf, cfg), ox, TOL_BF16, ELEM_BF16, 8, t)
        worst = max(worst, r)
        worst_e = max(worst_e, e)
        if t == 63:
            gst = S.to_host()
            r_state = rel(gst["gdn_state"], ost["gdn_state"])
            r_conv = rel(gst["conv1d_state"], ost["conv1d_state"])
            say(f"4B GDN after 64 steps: state rel {r_state:.2e}, conv rel {r_conv:.2e}")
            assert r_state < TOL_F32
            assert r_conv < TOL_F32
    gst = S.to_host()
    say(f"4B GDN: worst output rel {worst:.2e}, element error {worst_e:.3f} RMS; after 256 steps state rel "
        f"{rel(gst['gdn_state'], ost['gdn_state']):.2e}")


def test_full_layer_4b_bf16_64_steps_from_4096(rt, gen):
    """Config 3: 64 steps at cache_pos 4096..4159 over a prefilled bf16 cache;
    every output within the bf16 tolerance, KV placement exact."""
    steps = 64
    w = workloads.full_layer_4b(gen, steps=steps)
    cfg, layer, kv = w["cfg"], w["layer"], w["kv"]
    start = w["start"]
    cap = kv["k"].shape[0]
    kv["k"][start:] = NAN_BF16
    kv["v"][start:] = NAN_BF16
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    scr = rt.FullScratchDev(cfg, cap)
    inv = rt.inv_freq_dev(cfg)
    inv_h = O.rope_inv_freq(cfg.rope_theta, cfg.rotary_dim)
    okv = {"k": kv["k"].copy(), "v": kv["v"].copy()}
    outs = []
    worst = worst_e = 0.0
    for i, x in enumerate(w["xs"]):
        t = start + i
        if i % 16 == 0:
            say(f"4B full attention at cache_pos {t}")
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), t)
        ox, okv, _ = O.forward_full_attention(cfg, layer, okv, inv_h, x, t)
        torch.cuda.synchronize()
        g = rt.act_to_f32(scr.t["x_out"], cfg)
        outs.append(g.copy())
        r, e = check(g, ox, TOL_BF16, ELEM_BF16, 8, t)
        worst = max(worst, r)
        worst_e = max(worst_e, e)
    say(f"4B full attention: worst output rel {worst:.2e}, element error {worst_e:.3f} RMS")
    after = KVd.to_host()
    for side in ("k", "v"):
        assert np.array_equal(after[side][:start], kv[side][:start])          # prefill untouched
        assert np.all(after[side][start + steps:] == NAN_BF16)                # beyond: untouched
        assert rel(O.bf16_to_f64(after[side][start:start + steps]),
                   O.bf16_to_f64(okv[side][start:start + steps])) < TOL_BF16

    # device-side position (the graph-replay entry point) gives the same layer
    KV2 = rt.KvCacheDev(kv)
    scr2 = rt.FullScratchDev(cfg, cap)
    pos = torch.tensor([start], dtype=torch.int32, device="cuda")
    for i, x in enumerate(w["xs"]):
        if i % 16 == 0:
            say(f"4B full attention, device position {start + i}")
        rt.forward_full_attention(cfg, Ld, scr2, KV2, inv, pos, rt.to_dev(x), None)
        torch.cuda.synchronize()
        assert rel(rt.act_to_f32(scr2.t["x_out"], cfg), outs[i]) < 1e-5
        pos += 1
    assert np.array_equal(KV2.to_host()["k"], after["k"])


def test_out_of_range_device_position_touches_nothing(rt, gen):
    """A device position outside the cache writes no KV row, gives a zero
    attention output and sets the position bit of the caller's status word;
    a position inside leaves the word clear."""
    from hybrid_decode_amd import binding as B
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, "gpu.oor")
    kv = synth.kv_cache(gen, cfg, "gpu.oor", 8, 8)
    Ld, KVd = rt.FullLayerDev(layer), rt.KvCacheDev(kv)
    scr = rt.FullScratchDev(cfg, 8)
    inv = rt.inv_freq_dev(cfg)
    x = rt.to_dev(gen.act("gpu.oor.x", (256,), "f32"))
    for p in (8, -1, 1 << 20):
        say(f"device position {p} with capacity 8")
        scr.t["status"].zero_()
        scr.t["gated_attn"].fill_(1.0)
        pos = torch.tensor([p], dtype=torch.int32, device="cuda")
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, x, None)
        torch.cuda.synchronize()
        h = KVd.to_host()
        assert np.array_equal(h["k"], kv["k"]) and np.array_equal(h["v"], kv["v"])
        assert int(scr.t["status"].cpu()[0]) == B.Q35_STATUS_POS_RANGE
        assert torch.count_nonzero(scr.t["gated_attn"]).item() == 0
    say("device position 7 with capacity 8")
    scr.t["status"].zero_()
    kv2 = synth.kv_cache(gen, cfg, "gpu.oor", 8, 7)
    KV2 = rt.KvCacheDev(kv2)
    rt.forward_full_attention(cfg, Ld, scr, KV2, inv, torch.tensor([7], dtype=torch.int32, device="cuda"),
                              x, None)
    torch.cuda.synchronize()
    assert int(scr.t["status"].cpu()[0]) == 0
