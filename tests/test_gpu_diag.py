"""The diagnostic register-only MFMA loop (lmhead_diag_mfma_loop) that the
benchmark times beside the GEMMs.  All-ones operands: every thread's output has
a closed form, 16 per MFMA per chain (all-ones 32x32x16 products), 8 chains, so
every element must equal 128 * iters exactly.  Random operands: each chain
cycles through products P1, P2, -P1, -P2 whose partial sums are exact in FP32,
so the output is exactly 0 after a multiple of 4 rounds and depends only on
iters % 4 otherwise (a dropped or repeated MFMA breaks both)."""
import pytest
import torch

import lm_head_fp32_amd as lmh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


@pytest.mark.parametrize("iters,n_wg", [(0, 3), (1, 1), (1000, 64), (100000, 512)])
def test_mfma_loop_closed_form(iters, n_wg):
    sink = torch.full((n_wg * 256,), -1.0, dtype=torch.float32, device="cuda")
    lmh.lmhead_diag_mfma_loop(iters, n_wg, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 128.0 * iters).item()


@pytest.mark.parametrize("n_wg", [1, 512])
def test_mfma_loop_random_cancels(n_wg):
    outs = {}
    for iters in (0, 1, 2, 3, 4, 5, 6, 7, 4000, 4001, 4002, 4003):
        sink = torch.full((n_wg * 256,), -1.0, dtype=torch.float32, device="cuda")
        lmh.lmhead_diag_mfma_loop(iters, n_wg, sink, operands="random")
        torch.cuda.synchronize()
        outs[iters] = sink.cpu()
    for iters, v in outs.items():
        assert torch.isfinite(v).all()
        if iters % 4 == 0:
            assert torch.all(v == 0.0).item(), iters
        else:
            assert torch.equal(v, outs[iters % 4]), iters
            assert (v != 0.0).float().mean().item() > 0.9  # random data, not cancelled
    # lanes hold different operands
    assert torch.unique(outs[1]).numel() > n_wg * 256 // 2
