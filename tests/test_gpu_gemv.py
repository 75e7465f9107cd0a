"""GPU parity of the int8 group-64 GEMV kernel family against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import TOL_GEMV, TOL_GEMV_F16, rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    from hybrid_decode_amd import runtime
    runtime.kernels(0)
    return runtime


# (K, rows): rows a multiple of the rows-per-wave group at that K
SHAPES = [(128, 16), (256, 16), (512, 8), (2560, 8), (4096, 4), (9216, 4)]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("K,rows", SHAPES)
def test_one_hot_gemv_returns_dequantised_columns_bit_exact(rt, gen, K, rows, act):
    from hybrid_decode_amd import binding as B
    w = gen.quant(f"gpu.onehot.{K}", rows, K)
    dense = O.dequant(w)
    W = rt.QuantWeightDev(w)
    for j in sorted({0, 1, 15, 16, 63, 64, 65, K // 2, K - 1}):
        say(f"one-hot GEMV ({act}) K={K} rows={rows} column={j}")
        x = torch.zeros(K, dtype=torch.float32, device="cuda")
        x[j] = 1.0
        y = torch.empty(rows, dtype=torch.float32, device="cuda")
        B.q35_gemv(rt.kernels(), W.struct, x.data_ptr(), y.data_ptr(),
                   B.Q35_ACT_F32 if act == "f32" else B.Q35_ACT_BF16, rt.stream_ptr())
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), dense[:, j]), (K, j)


@pytest.mark.parametrize("act,tol", [("f32", TOL_GEMV), ("bf16", TOL_GEMV_F16)])
@pytest.mark.parametrize("K,rows", [(2560, 1024), (4096, 320), (9216, 256), (512, 130), (128, 200)])
def test_random_gemv_matches_oracle(rt, gen, K, rows, act, tol):
    from hybrid_decode_amd import binding as B
    say(f"random GEMV ({act}) K={K} rows={rows}")
    w = gen.quant(f"gpu.gemv.{K}.{rows}", rows, K)
    x = gen.normal_f32(f"gpu.gemv.x.{K}", (K,))
    W = rt.QuantWeightDev(w)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    B.q35_gemv(rt.kernels(), W.struct, rt.to_dev(x).data_ptr(), y.data_ptr(),
               B.Q35_ACT_F32 if act == "f32" else B.Q35_ACT_BF16, rt.stream_ptr())
    torch.cuda.synchronize()
    ref = O.as_qm(w) @ x.astype(np.float64)
    r = rel(y.cpu().numpy(), ref)
    say(f"  rel {r:.2e}")
    assert r < tol


def test_lm_head_full_vocab_argmax_and_embedding(rt, gen):
    """The int8 lm_head at the 4B shape (248 320 x 2560): every logit, the greedy
    token, the position increment, the history write and the next embedding."""
    from hybrid_decode_amd import binding as B
    cfg = synth.qwen3_5_4b("bf16")
    c = rt.cfg_struct(cfg)
    say("lm_head: generating 248320 x 2560 weights")
    lm = gen.quant("gpu.lm_head", cfg.vocab, cfg.hidden)
    fnorm = gen.norm_weight("gpu.final_norm", cfg.hidden)
    embed = gen.normal_bf16("gpu.embed", (cfg.vocab, cfg.hidden))
    x = gen.act("gpu.lm.x", (cfg.hidden,), "bf16")
    W = rt.QuantWeightDev(lm)
    d_fn, d_emb, d_x = rt.to_dev(fnorm), rt.to_dev(embed), rt.to_dev(x)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    ws = torch.zeros(B.q35_lm_head_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    tokens = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    positions = torch.tensor([100], dtype=torch.int32, device="cuda")
    history = torch.full((8,), -1, dtype=torch.int32, device="cuda")
    x_next = rt.act_empty(cfg, cfg.hidden)
    for rep in range(2):  # the second call checks the workspace counter was left at zero
        say(f"lm_head call {rep}")
        B.q35_lm_head_argmax(rt.kernels(), c, d_fn.data_ptr(), W.struct, d_x.data_ptr(),
                             logits.data_ptr(), ws.data_ptr(), ws.numel(), tokens.data_ptr(),
                             positions.data_ptr(), history.data_ptr(), 8, 98,
                             d_emb.data_ptr(), x_next.data_ptr(), rt.stream_ptr())
    torch.cuda.synchronize()
    g = logits.cpu().numpy()
    h = O.rms_norm(O.act_to_f64(x, "bf16"), fnorm, cfg.rms_eps)
    ref = np.empty(cfg.vocab)
    for r0 in range(0, cfg.vocab, 16384):
        blk = {k: v[r0:r0 + 16384] for k, v in lm.items()}
        ref[r0:r0 + 16384] = O.dequant(blk).astype(np.float64) @ h
    r = rel(g, ref)
    say(f"lm_head logits rel {r:.2e}")
    assert r < TOL_GEMV_F16
    tok = int(tokens.cpu()[0])
    assert tok == int(np.argmax(g))                       # argmax of its own logits, exactly
    top2 = np.sort(ref)[-2:]
    if top2[1] - top2[0] > 1e-4 * abs(top2[1]):
        assert tok == O.greedy(ref)
    assert int(positions.cpu()[0]) == 102
    hist = history.cpu().numpy()
    assert hist[2] == tok and hist[3] == tok and np.all(hist[[0, 1, 4, 5, 6, 7]] == -1)
    assert np.array_equal(rt.act_to_host(x_next, cfg), embed[tok])
