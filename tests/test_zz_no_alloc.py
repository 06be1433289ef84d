"""lmhead_dgrad_noalloc, the V-split dgrad whose FP32 partials live in the
library's fixed per-GPU scratch array instead of a caller workspace, against
lmhead_dgrad_ws with the same split, through the C ABI.  The two run the same
kernels in the same order, so dX must agree bit for bit (above the 1e-5 * S
bar of the GEMMs).  Two calls in a row, the second smaller, show that a call
reads only partials it wrote itself (the array keeps the last call's
contents); the first call fills the whole 64 MiB array."""
import numpy as np
import pytest
import torch

import lm_head_fp32_amd as lmh
import oracle
import workloads
from gpu_util import assert_gemm_close, dev_bf16, host_f32, padded_out, padding_untouched

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


def _say(*a):
    print(*a, flush=True)


def _ws_and_noalloc(dl, W, M, K, V, splits, dtype):
    need = lmh.lmhead_dgrad_workspace_bytes(M, K, V, splits)
    assert 0 < need <= lmh.DGRAD_NOALLOC_MAX_BYTES
    ws = torch.full((need // 4,), float("nan"), device="cuda")
    ref = padded_out(M, K, K + 8, dtype)
    got = padded_out(M, K, K + 8, dtype)
    lmh.lmhead_dgrad(dl, W, dX=ref, splits=splits, workspace=ws)
    lmh.lmhead_dgrad_noalloc(dl, W, got, splits=splits)
    torch.cuda.synchronize()
    assert padding_untouched(got)
    return ref, got


def test_noalloc_equals_workspace_path_two_calls():
    # call 1: M=1024 K=8192 V=32768 (the benchmark's dgrad), default split in
    # two: 2 x 1024 x 8192 FP32 partials = the whole 64 MiB array
    rng = np.random.default_rng(workloads.SEED + 71)
    M, K, V = 1024, 8192, 32768
    dl_bits = workloads.normal_bf16(rng, (M, V), 1e-3)
    W_bits = workloads.normal_bf16(rng, (V, K), 0.02)
    dl, W = dev_bf16(dl_bits), dev_bf16(W_bits)
    assert lmh.lmhead_dgrad_workspace_bytes(M, K, V) == lmh.DGRAD_NOALLOC_MAX_BYTES
    _say("noalloc call 1: 1024x8192x32768, fp32 and bf16 dX")
    for dtype in (torch.float32, torch.bfloat16):
        ref, got = _ws_and_noalloc(dl, W, M, K, V, 0, dtype)
        assert torch.equal(ref.contiguous().view(torch.int16 if dtype == torch.bfloat16
                                                 else torch.int32),
                           got.contiguous().view(torch.int16 if dtype == torch.bfloat16
                                                 else torch.int32))
    dx32 = lmh.lmhead_dgrad_noalloc(dl, W, torch.empty(M, K, device="cuda"))
    torch.cuda.synchronize()
    rows = np.array([0, 511, 1023])
    r, S = oracle.dgrad(dl_bits, W_bits, rows=rows)
    assert_gemm_close(host_f32(dx32)[rows], r, S, 1e-5, "noalloc dgrad")
    del dl, W
    # call 2, smaller: ragged integers, 16 parts, M=130 K=520 V=4100; the
    # array still holds call 1's partials
    dl_bits, W_bits = workloads.integer_operands([(130, 4100), (4100, 520)], seed=72)
    dl, W = dev_bf16(dl_bits, 4104), dev_bf16(W_bits, 528)
    _say("noalloc call 2: integers 130x520x4100, 16 parts")
    ref, got = _ws_and_noalloc(dl, W, 130, 520, 4100, 16, torch.float32)
    assert torch.equal(ref.contiguous().view(torch.int32), got.contiguous().view(torch.int32))
    exact, _ = oracle.dgrad(dl_bits, W_bits)
    assert np.array_equal(host_f32(got).astype(np.float64), exact)


def test_noalloc_rejects_oversized_and_runs_unsplit():
    # 4 parts of 1024 x 8192 need 128 MiB: refused before anything runs
    assert lmh.lmhead_dgrad_workspace_bytes(1024, 8192, 32768, 4) > lmh.DGRAD_NOALLOC_MAX_BYTES
    dl = torch.zeros((1024, 32768), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32768, 8192), dtype=torch.bfloat16, device="cuda")
    dX = torch.full((1024, 8192), float("nan"), device="cuda")
    with pytest.raises(lmh.LmheadError) as e:
        lmh.lmhead_dgrad_noalloc(dl, W, dX, splits=4)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.isnan(dX).all().item()
    # a shape that runs unsplit is lmhead_dgrad (no scratch)
    dl_bits, W_bits = workloads.integer_operands([(33, 72), (72, 40)], seed=73)
    out = torch.empty((33, 40), device="cuda")
    lmh.lmhead_dgrad_noalloc(dev_bf16(dl_bits), dev_bf16(W_bits), out, splits=1)
    torch.cuda.synchronize()
    exact, _ = oracle.dgrad(dl_bits, W_bits)
    assert np.array_equal(host_f32(out).astype(np.float64), exact)
