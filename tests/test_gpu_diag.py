"""The diagnostic register-only MFMA loop (lmhead_diag_mfma_loop) that the
benchmark times beside the GEMMs: every thread's output has a closed form,
16 per MFMA per chain (all-ones 32x32x16 products), 8 chains, so every
element must equal 128 * iters exactly."""
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
