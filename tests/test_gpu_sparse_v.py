"""GPU parity of the sparse-V gate of the quantised KV formats (full_attention.rs
page, Turbo branches: a threshold below which a position's value row is left
out; 1e-3 unless overridden, 0 disables it).

For every quantised format the tiny fp32 layer runs one step at cache
position 512 with the threshold 0, 1e-3, 0.05 and 0.3; the attention tap is
compared with the oracle's attention over the cache as stored, with the
kernel's own query and the same threshold.  The oracle leaves out every row
whose weight relative to the largest is below the threshold; the kernel
compares against its running maximum and needs every lane of a wave to agree,
so it leaves out a subset of those rows.  The difference per head is therefore
bounded in L2 norm by the dropped weight times the dropped rows' norms (the
output rotation is orthonormal), on top of the fp32 tolerance; at threshold 0
the two are equal within it, and at 0.3 the gate must have dropped something.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import TOL_F32, check_gated_attention, gated_attention_ref, rel, say

pytestmark = pytest.mark.gpu

FORMATS = ["turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def _cache(gen, cfg, fmt, cap, filled):
    if fmt == "turbo8":
        return synth.kv_cache_turbo8(gen, cfg, "gpu.sv.turbo8", cap, filled)
    return synth.kv_cache_lm(gen, cfg, f"gpu.sv.{fmt}", cap, filled, fmt)


@pytest.mark.parametrize("fmt", FORMATS)
def test_sparse_v_gate_within_the_dropped_weight(rt, gen, fmt):
    cfg = synth.tiny("f32")
    layer = synth.full_layer(gen, cfg, f"gpu.sv.{fmt}")
    start = 512
    cap = start + 8
    x = gen.act(f"gpu.sv.{fmt}.x", (cfg.hidden,), "f32")
    Ld = rt.FullLayerDev(layer)
    inv = rt.inv_freq_dev(cfg)
    Hq, D = cfg.num_heads, cfg.head_dim
    rep = Hq // cfg.num_kv_heads
    attn = {}
    for tau in (0.0, 1e-3, 0.05, 0.3):
        kv = _cache(gen, cfg, fmt, cap, start)
        KVd = rt.KvCacheDev(kv, sparse_v=tau)
        scr = rt.FullScratchDev(cfg, cap, taps=True)
        pos = torch.tensor([start], dtype=torch.int32, device="cuda")
        say(f"{fmt}: sparse_v {tau}")
        rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), start)
        torch.cuda.synchronize()
        after = KVd.to_host()
        q = scr.t["q_norm_out"].cpu().numpy().astype(np.float64).reshape(Hq, D)
        g = scr.t["attn_out"].cpu().numpy().astype(np.float64).reshape(Hq, D)
        e, b, ndrop = check_gated_attention(g, fmt, q, after, start + 1, tau, rep, TOL_F32)
        say(f"  oracle drops {ndrop} of {Hq * (start + 1)} (row, head) pairs; "
            f"max error {e:.2e} of the norm, bound {b:.2e}")
        if tau == 0.0:
            assert ndrop == 0
            assert rel(g, gated_attention_ref(fmt, q, after, start + 1, 0.0)) < TOL_F32
        attn[tau] = g
    # the gate did drop rows: its output moved away from the exact one
    assert rel(attn[0.3], attn[0.0]) > 1e-6
