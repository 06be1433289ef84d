"""The full LM-head step at its full size, M=4096 tokens, K=16384, V=131072
(x ~ N(0,1), W ~ N(0, 0.01^2)), in the launch configuration the benchmark
uses, checked on sampled outputs against the FP64 oracle.

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
from gpu_util import assert_gemm_close, assert_loss_close, dev_bf16, host_f32

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
