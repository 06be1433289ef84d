"""The LM-head chain against the FP64 oracle chain built from x and W:
at M=128, K=4096, V=32768 with 6 ignored rows (every output), and the full
step at its full size, M=4096 tokens, K=16384, V=131072 (x ~ N(0,1),
W ~ N(0, 0.01^2)), in the launch configuration the benchmark uses, on
sampled outputs.

  logits (FP32) -> CE forward -> mean -> CE backward (BF16 dlogits)
  dgrad dX = dlogits . W  and  wgrad dW = dlogits^T . x  (FP32 accumulate)

The oracle never takes a GPU result as input: the chain's logits and CE are
checked on sampled rows from x and W; dgrad and wgrad are checked on their
own seeded BF16 dlogits of the same shape and magnitude.  Properties that
hold at any size are checked on the whole outputs (no NaN/inf, gradient rows
sum to zero, BF16 gradients = nearest-even rounding of the FP32 ones)."""
import numpy as np
import pytest
import torch

import lm_head_fp32_amd as lmh
import oracle
import workloads
from gpu_util import assert_gemm_close, assert_loss_close, dev_bf16, dev_i32, host_f32

pytestmark = pytest.mark.gpu

M, K, V = 4096, 16384, 131072
ROWS = np.array([0, 1, 2047, 2048, 4095])


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


def _say(*a):
    print(*a, flush=True)


def test_chain_lmhead_128_against_oracle_chain():
    """M=128, K=4096, V=32768, x ~ N(0,1), W ~ N(0, 0.02^2), targets uniform
    with 6 rows (5 %) ignored: FP32 logits -> CE forward -> mean -> FP32
    backward with dloss = 1/n_valid, every output against the oracle chain
    (logits from x and W in FP64, rounded once to FP32; the CE of those).

    The GPU's logits differ from the oracle's by at most 1e-5 * S (checked);
    a row whose logits move by at most D moves its loss by at most 2 D and its
    gradient by at most 2 D p_j dloss (to first order), so each row is held to
    the CE tolerances plus that propagated error, with D the row's measured
    largest logit difference."""
    inp = workloads.lmhead_128()
    Mc, Vc = inp.x.shape[0], inp.W.shape[0]
    ign = inp.target == workloads.IGNORE_INDEX
    assert ign.sum() == 6
    _say("chain lmhead_128")
    x, W, t = dev_bf16(inp.x), dev_bf16(inp.W), dev_i32(inp.target)
    logits = lmh.lmhead_logits(x, W, out_dtype="fp32")
    loss, st = lmh.lmhead_xent_fwd(logits, t)
    mean, inv = lmh.lmhead_xent_mean(loss, t)
    g = lmh.lmhead_xent_bwd(logits, st, t, inv)
    torch.cuda.synchronize()
    L, S = oracle.logits(inp.x, inp.W)
    zh = host_f32(logits)
    assert_gemm_close(zh, L, S, 1e-5, "logits")
    L32 = L.astype(np.float32)
    D = np.abs(zh.astype(np.float64) - L32.astype(np.float64)).max(axis=1)
    ref = oracle.xent_fwd(L32, inp.target, -100)
    m_ref, inv_ref, nv = oracle.xent_mean(ref[:, 3], inp.target, -100)
    assert nv == Mc - 6
    assert host_f32(inv)[0] == np.float32(inv_ref)
    sh, lh = host_f32(st), host_f32(loss)
    assert np.array_equal(lh, sh[:, 3])
    assert np.all(lh[ign] == 0.0) and np.all(sh[ign, 2] == 0.0)
    bound = 1e-5 * np.maximum(np.abs(ref[:, 3]), 1.0) + 2.0 * D
    assert np.all(np.abs(lh - ref[:, 3]) <= bound)
    assert np.all(np.abs(sh[:, 0] - ref[:, 0]) <= D)            # max moves by at most D
    assert abs(float(host_f32(mean)[0]) - m_ref) <= 1e-5 * abs(m_ref) + 2.0 * D.max()
    g_ref = oracle.xent_bwd(L32, inp.target, -100, inv_ref)
    gh = host_f32(g).astype(np.float64)
    assert np.all(gh[ign] == 0.0)
    p = np.abs(g_ref) / inv_ref                                  # p_j, or 1 - p_y at the target
    gbound = 1e-6 + 2.01 * inv_ref * D[:, None] * np.maximum(p, 1e-30) * 1.01 + 1e-12
    err = np.abs(gh - g_ref)
    assert np.all(err <= np.maximum(gbound, 1e-6)), float(err.max())
    # and relative to each entry: the FP32 kernel's own error (argument and
    # exponential rounding, about 2^-23 |z - m| + a few ulp) plus the
    # propagated logit difference
    rel = (2e-5 + 2.02 * D[:, None]) * np.abs(g_ref) + 1e-15
    assert np.all(err[~ign] <= rel[~ign]), float((err / (np.abs(g_ref) + 1e-30))[~ign].max())
    assert np.abs(gh.sum(axis=1)).max() <= 1e-5 * inv_ref + 1e-9


def test_step_4096_logits_and_cross_entropy():
    _say("step 4096: generating x, W")
    inp = workloads.step_4096()
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    t = torch.from_numpy(inp.target).cuda()
    _say("step 4096: logits -> CE")
    logits = lmh.lmhead_logits(x, W, out_dtype="fp32")
    loss, st = lmh.lmhead_xent_fwd(logits, t)
    mean, inv = lmh.lmhead_xent_mean(loss, t)
    gb = lmh.lmhead_xent_bwd(logits, st, t, inv, grad_dtype="bf16")
    g32 = lmh.lmhead_xent_bwd(logits, st, t, inv)
    torch.cuda.synchronize()
    assert torch.isfinite(logits).all().item() and torch.isfinite(g32).all().item()
    assert torch.equal(gb.view(torch.int16), g32.to(torch.bfloat16).view(torch.int16))
    rs = g32.double().sum(dim=1).abs().max().item()
    assert rs <= 1e-5 * float(host_f32(inv)[0]) + 1e-9
    # sampled rows against the oracle (logits from x and W, CE from those)
    L, S = oracle.logits(inp.x, inp.W, rows=ROWS)
    assert_gemm_close(host_f32(logits[torch.from_numpy(ROWS).cuda()]), L, S, 1e-5, "logits")
    ref = oracle.xent_fwd(L.astype(np.float32), inp.target[ROWS], -100)
    bound = 2e-5 * S.max(axis=1) + 1e-5 * np.abs(ref[:, 3]) + 1e-6
    assert np.all(np.abs(host_f32(loss)[ROWS] - ref[:, 3]) <= bound)
    assert host_f32(inv)[0] == np.float32(1.0 / M)       # no ignored rows here
    g_ref = oracle.xent_bwd(L.astype(np.float32), inp.target[ROWS], -100, 1.0 / M)
    gs = host_f32(g32[torch.from_numpy(ROWS).cuda()]).astype(np.float64)
    # the gradient's error follows the logits' (|dg| <= dloss * |dlogit|-scale)
    assert np.abs(gs - g_ref).max() <= 4e-5 * S.max() / M + 1e-9
    assert_loss_close(host_f32(mean), [float(np.mean(host_f32(loss), dtype=np.float64))], 1e-5, "mean")


def test_step_4096_dgrad_wgrad():
    _say("step 4096: generating dlogits, W, x")
    rng = np.random.default_rng(workloads.SEED + 41)
    dl_bits = workloads.normal_bf16(rng, (M, V), 1.0 / (M * 64))
    inp = workloads.step_4096()
    dl, W, x = dev_bf16(dl_bits), dev_bf16(inp.W), dev_bf16(inp.x)
    _say("step 4096: dgrad, wgrad")
    dx16 = lmh.lmhead_dgrad(dl, W)                        # BF16 dX, the default
    dx = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32")
    dw = lmh.lmhead_wgrad(dl, x)
    torch.cuda.synchronize()
    assert torch.isfinite(dx).all().item() and torch.isfinite(dw).all().item()
    assert torch.equal(dx16.view(torch.int16), dx.to(torch.bfloat16).view(torch.int16))
    ref, S = oracle.dgrad(dl_bits, inp.W, rows=ROWS)
    assert_gemm_close(host_f32(dx)[ROWS], ref, S, 1e-5, "dgrad")
    vrows = np.array([0, 1, 65535, 65536, 131071])
    ref, S = oracle.wgrad(dl_bits, inp.x, rows=vrows)
    assert_gemm_close(host_f32(dw[torch.from_numpy(vrows).cuda()]), ref, S, 1e-5, "wgrad")
