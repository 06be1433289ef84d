"""Seeded random-shape parity sweep through the C ABI: the logits GEMM (FP32
and BF16 epilogues), dgrad and wgrad on integer operands in [-8, 8], which
are exact in FP32 at these sizes (every product and partial sum is an integer
below 2^24), so each output must equal the FP64 oracle bit for bit; and the
CE forward and backward, and the single-read forward + backward, on those
exact logits scaled by 1/64 (a power of two, so still exact), with 10 % of
rows ignored, against the oracle to the usual tolerances (m and X_y
bit-exact, loss 1e-5 relative, gradient 1e-6 absolute).

Shapes mix single rows, ragged tile edges (M, V not multiples of the tiles,
K any multiple of 8) and padded leading dimensions, so the kernels' edge
paths are exercised at sizes the oracle checks in full.  Each case prints its
shape before it runs."""
import numpy as np
import pytest
import torch

import lm_head_fp32_amd as lmh
import oracle
import workloads
from gpu_util import assert_loss_close, dev_bf16, dev_f32, dev_i32, host_bits, host_f32

pytestmark = pytest.mark.gpu

SMALL = workloads.random_shapes(24, 20251, (1, 3, 16, 17, 63, 100, 128, 129, 255, 256, 257, 300, 511),
                                (1, 7, 64, 100, 255, 256, 257, 1000, 2049), 200)
LARGE = workloads.random_shapes(4, 20252, (300, 512, 700, 1024, 1100), (256, 1000, 4100, 5000), 300)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


def _round_up(v, m):
    return (v + m - 1) // m * m


@pytest.mark.parametrize("case", range(len(SMALL) + len(LARGE)))
def test_random_shape_parity(case):
    c = (SMALL + LARGE)[case]
    M, K, V = c["M"], c["K"], c["V"]
    print(f"random shape case {case}: {c}", flush=True)
    xb, Wb, gb = workloads.integer_operands([(M, K), (V, K), (M, V)], seed=30000 + case)
    x, W = dev_bf16(xb, K + c["pad_x"]), dev_bf16(Wb, K + c["pad_w"])
    z = lmh.lmhead_logits(x, W, out_dtype="fp32")
    zb = lmh.lmhead_logits(x, W, out_dtype="bf16")
    g = dev_bf16(gb, _round_up(V, 8) + c["pad_g"])
    dX = lmh.lmhead_dgrad(g, W, dx_dtype="fp32")
    dW = lmh.lmhead_wgrad(g, x)
    torch.cuda.synchronize()
    L, _ = oracle.logits(xb, Wb)
    assert np.array_equal(host_f32(z).astype(np.float64), L)
    assert np.array_equal(host_bits(zb), oracle.round_bf16(L))
    Dx, _ = oracle.dgrad(gb, Wb)
    Dw, _ = oracle.wgrad(gb, xb)
    assert np.array_equal(host_f32(dX).astype(np.float64), Dx)
    assert np.array_equal(host_f32(dW).astype(np.float64), Dw)

    zz = (L / 64.0).astype(np.float32)
    t = workloads.uniform_targets(M, V, 0.1, seed=40000 + case)
    zd = dev_f32(zz, _round_up(V, 4) + c["pad_z"])
    td = dev_i32(t)
    loss, st = lmh.lmhead_xent_fwd(zd, td)
    grad = lmh.lmhead_xent_bwd(zd, st, td, torch.full((1,), 0.25, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.xent_fwd(zz, t)
    stg = host_f32(st).astype(np.float64)
    assert np.array_equal(stg[:, 0], ref[:, 0])
    assert np.array_equal(stg[:, 2], ref[:, 2])
    assert_loss_close(stg[:, 3], ref[:, 3])
    assert_loss_close(host_f32(loss), ref[:, 3])
    gref = oracle.xent_bwd(zz, t, -100, 0.25)
    assert np.max(np.abs(host_f32(grad).astype(np.float64) - gref), initial=0.0) <= 1e-6

    # the single-read kernel on the same logits: FP32 and BF16 gradients
    dl = torch.full((1,), 0.25, device="cuda")
    floss, fst, fg = lmh.lmhead_xent_fused(zd, td, dl)
    _, fst16, fg16 = lmh.lmhead_xent_fused(zd, td, dl, grad_dtype="bf16")
    torch.cuda.synchronize()
    fs = host_f32(fst).astype(np.float64)
    assert np.array_equal(fs[:, 0], ref[:, 0])
    assert np.array_equal(fs[:, 2], ref[:, 2])
    assert_loss_close(fs[:, 3], ref[:, 3])
    assert_loss_close(host_f32(floss), ref[:, 3])
    assert torch.equal(fst.view(torch.int32), fst16.view(torch.int32))
    assert np.max(np.abs(host_f32(fg).astype(np.float64) - gref), initial=0.0) <= 1e-6
    assert torch.equal(fg16.view(torch.int16), fg.to(torch.bfloat16).view(torch.int16))
