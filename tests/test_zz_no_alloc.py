"""The lm_head entry point that allocates nothing (fixed per-GPU workspace)
against the one that takes a caller workspace: two calls in a row, the second
with a smaller vocabulary, each bit-identical to the workspace path."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


def _case(rt, gen, vocab, tag):
    cfg = dataclasses.replace(synth.qwen3_5_4b("bf16"), vocab=vocab)
    lm = gen.quant(f"noalloc.{tag}.lm", vocab, cfg.hidden)
    embed = gen.normal_bf16(f"noalloc.{tag}.embed", (vocab, cfg.hidden))
    fn = gen.norm_weight(f"noalloc.{tag}.fn", cfg.hidden)
    x = gen.act(f"noalloc.{tag}.x", (cfg.hidden,), "bf16")
    return cfg, rt.QuantWeightDev(lm), rt.to_dev(embed), rt.to_dev(fn), rt.to_dev(x)


def _run(rt, B, cfg, lm, embed, fn, x, noalloc, pos0):
    c = rt.cfg_struct(cfg)
    k = rt.kernels(0)
    logits = torch.full((cfg.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    tokens = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    positions = torch.tensor([pos0], dtype=torch.int32, device="cuda")
    history = torch.full((8,), -1, dtype=torch.int32, device="cuda")
    x_next = torch.zeros(cfg.hidden, dtype=torch.uint16, device="cuda")
    s = rt.stream_ptr()
    if noalloc:
        B.q35_lm_head_argmax_noalloc(k, c, fn.data_ptr(), lm.struct, x.data_ptr(), logits.data_ptr(),
                                     tokens.data_ptr(), positions.data_ptr(), history.data_ptr(), 8,
                                     pos0 - 3, embed.data_ptr(), x_next.data_ptr(), s)
    else:
        nb = B.q35_lm_head_workspace_bytes(c)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        B.q35_lm_head_argmax(k, c, fn.data_ptr(), lm.struct, x.data_ptr(), logits.data_ptr(),
                             ws.data_ptr(), nb, tokens.data_ptr(), positions.data_ptr(),
                             history.data_ptr(), 8, pos0 - 3, embed.data_ptr(), x_next.data_ptr(), s)
    torch.cuda.synchronize()
    return (logits.cpu().numpy(), int(tokens.cpu()[0]), int(positions.cpu()[0]),
            history.cpu().numpy(), x_next.cpu().numpy())


def test_noalloc_lm_head_matches_the_workspace_path_twice(rt, gen):
    from hybrid_decode_amd import binding as B
    for vocab, tag in ((248_320, "big"), (4_096, "small")):
        say(f"no-alloc lm_head, vocab {vocab}")
        cfg, lm, embed, fn, x = _case(rt, gen, vocab, tag)
        ref = _run(rt, B, cfg, lm, embed, fn, x, False, 100)
        got = _run(rt, B, cfg, lm, embed, fn, x, True, 100)
        assert np.array_equal(got[0], ref[0])               # logits, bit for bit
        assert got[1] == ref[1] == int(np.argmax(ref[0]))  # token
        assert got[2] == ref[2] == 101                      # position advanced
        assert np.array_equal(got[3], ref[3]) and got[3][3] == got[1]
        assert np.array_equal(got[4], ref[4])               # next embedding row
        say(f"  token {got[1]}")
