"""GPU parity of the matrix-core tiles of decode attention over the quantised KV
formats (full_attention.rs page, the Turbo branches of `attention_decode`, with
the sparse-V gate; mod.rs, the Turbo and Bf16K + TurboNV cache formats).

At head dimension 128 or 256, once a split-K chunk holds at least 64 rows, the
partial kernel decodes the chunk's rows 64 at a time into LDS (E4M3 codes,
codebook levels or bf16 keys) and runs the scores and the weighted value sum
on the matrix cores.  The cases below pick
cache lengths whose chunks hold one to three such tiles with ragged tails,
and positions whose row falls inside a later tile of its chunk (the appended
row enters from the values as stored).  For each, one layer step runs with the
gate off, at its default and at 0.3; the attention tap is compared with the
oracle's attention over the cache as stored, with the kernel's own query: at
threshold 0 within TOL_TILE per head and as a whole, and element by element
within one fp32 step plus ELEM_F32 times the RMS of the oracle's output;
otherwise within TOL_TILE plus the weight of the rows the oracle's gate drops
(the kernel drops a subset of those).

TOL_TILE: the tiles hold q, k, v and the weights p as f16 (each rounded once,
unit roundoff 2^-11, with fp32 accumulation), where the bf16-activation
tolerance 2e-2 covers operands with unit roundoff 2^-8; scaled by the ratio of
the two, 2.5e-3.  A CPU emulation of these roundings on the Lloyd-Max caches
below (scores spread wider than on the Turbo8 ones) gives up to 8e-4 of the
norm with unit-variance queries.

Layer: hidden 256 (the projections are not what is tested here), the head
geometry of each case; cache rows drawn as in the other quantised-format tests
(Turbo8: every finite E4M3 code, bf16 scales U(1e-3, 1e-2); Lloyd-Max formats:
``synth.kv_cache_lm``).  Turbo8 runs every case below; each Lloyd-Max format
(three index widths, K in the format or in bf16) runs one case at each head
dimension.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from gpu_common import ELEM_F32, TOL_BF16, check, check_gated_attention, gated_attention_ref, rel, say

pytestmark = pytest.mark.gpu

TOL_TILE = TOL_BF16 / 8

# (head_dim, query heads, kv heads, rotary dims, positions)
#   256 / 16 / 4: chunks of 64 rows at position 8191 (one tile each), 152 rows
#                 at 19100 (pos at row 100: tile 1 of a 101-row chunk), 192 rows
#                 at 24575 (three tiles, pos the last row)
#   256 / 16 / 2: G = 8, chunks of 152 rows at 38900 (pos at row 140)
#   128 / 8 / 2:  chunks of 64 rows at 700 (eleven chunks, the last ragged),
#                 128 rows at 20000 (pos at row 32 of a chunk's first tile)
#   128 / 4 / 4:  G = 1 at 5000
CASES = [
    (256, 16, 4, 64, (8191, 19100, 24575)),
    (256, 16, 2, 64, (38900,)),
    (128, 8, 2, 32, (700, 20000)),
    (128, 4, 4, 32, (5000,)),
]
LM_FORMATS = ["turbo4", "turbo3", "turbo2", "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"]
LM_CASES = [(256, 16, 4, 64, (19100,)), (128, 8, 2, 32, (700,))]


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def _cfg(D, hq, hkv, rot):
    return replace(synth.tiny("f32"), num_heads=hq, num_kv_heads=hkv, head_dim=D, rotary_dim=rot)


def _cache(gen, cfg, fmt, name, cap, filled):
    if fmt == "turbo8":
        return synth.kv_cache_turbo8(gen, cfg, name, cap, filled)
    return synth.kv_cache_lm(gen, cfg, name, cap, filled, fmt)


@pytest.mark.parametrize("D,hq,hkv,rot,positions", CASES,
                         ids=[f"d{c[0]}_g{c[1] // c[2]}" for c in CASES])
def test_turbo8_tiles_match_the_oracle(rt, gen, D, hq, hkv, rot, positions):
    _run(rt, gen, "turbo8", D, hq, hkv, rot, positions)


@pytest.mark.parametrize("fmt", LM_FORMATS)
@pytest.mark.parametrize("D,hq,hkv,rot,positions", LM_CASES,
                         ids=[f"d{c[0]}_g{c[1] // c[2]}" for c in LM_CASES])
def test_lloyd_max_tiles_match_the_oracle(rt, gen, fmt, D, hq, hkv, rot, positions):
    _run(rt, gen, fmt, D, hq, hkv, rot, positions)


def _run(rt, gen, fmt, D, hq, hkv, rot, positions):
    cfg = _cfg(D, hq, hkv, rot)
    layer = synth.full_layer(gen, cfg, f"gpu.t8mf.d{D}.g{hq // hkv}")
    inv = rt.inv_freq_dev(cfg)
    Ld = rt.FullLayerDev(layer)
    rep = hq // hkv
    for start in positions:
        cap = start + 4
        x = gen.act(f"gpu.t8mf.d{D}.g{rep}.x{start}", (cfg.hidden,), "f32")
        attn = {}
        for tau in (0.0, 1e-3, 0.3):
            kv = _cache(gen, cfg, fmt, f"gpu.t8mf.{fmt}.d{D}.g{rep}.{start}", cap, start)
            KVd = rt.KvCacheDev(kv, sparse_v=tau)
            scr = rt.FullScratchDev(cfg, cap, taps=True)
            pos = torch.tensor([start], dtype=torch.int32, device="cuda")
            say(f"{fmt} tiles: D {D}, G {rep}, Hkv {hkv}, position {start}, sparse_v {tau}")
            rt.forward_full_attention(cfg, Ld, scr, KVd, inv, pos, rt.to_dev(x), start)
            torch.cuda.synchronize()
            after = KVd.to_host()
            q = scr.t["q_norm_out"].cpu().numpy().astype(np.float64).reshape(hq, D)
            g = scr.t["attn_out"].cpu().numpy().astype(np.float64).reshape(hq, D)
            assert np.all(np.isfinite(g))
            e, b, nd = check_gated_attention(g, fmt, q, after, start + 1, tau, rep, TOL_TILE)
            say(f"  error {e:.2e} of the norm (dropped-weight bound {b:.2e}, {nd} pairs dropped by the oracle)")
            if tau == 0.0:
                assert nd == 0
                # and element by element (fp32 output, as the other fp32 gates)
                check(g, gated_attention_ref(fmt, q, after, start + 1, 0.0), TOL_TILE, ELEM_F32, 24,
                      (fmt, D, rep, start))
            attn[tau] = g
            del KVd, scr
        assert rel(attn[0.3], attn[0.0]) > 1e-6   # the gate dropped rows
