"""GPU parity of the three GEMMs (logits, dgrad, wgrad) against the FP64
oracle, through the C ABI (via the thin binding).

Bar: bit-exact on integer operands (every FP32 partial sum is exact when
K * 8^2 < 2^24, Megatron-LM "Add mixed-precision (FP32) LM output logits",
section "Tests"); on random operands |gpu - L| <= 1e-5 * sum_k |x_k w_k|.
BF16 outputs are bit-exact on integers (round-to-nearest-even of the exact
value) and within 1e-5 * S plus half a BF16 spacing on random operands."""
import numpy as np
import pytest
import torch

import lm_head_fp32_amd as lmh
import oracle
import workloads
from gpu_util import (assert_gemm_close, dev_bf16, dev_f32, host_bits, host_f32, padded_out,
                      padding_untouched)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()  # fail loudly if the library is missing


def _say(*a):
    print(*a, flush=True)


def _padded_ld(n, mult):
    """A leading dimension past n (at least one element of padding) that is
    a multiple of mult elements (the 16-byte row alignment the C ABI asks)."""
    return (n + 2 * mult - 1) // mult * mult


def _f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------- logits

def test_logits_tiny_exact_fp32_and_bf16():
    """x [16 x 512], W [1024 x 512] integers in [-8, 8], seed 1234: FP32
    logits bit-exact; BF16 logits bit-exact to RNE of the exact value."""
    inp = workloads.tiny_exact()
    _say("tiny_exact logits")
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    out = lmh.lmhead_logits(x, W, out_dtype="fp32")
    outb = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    L, _ = oracle.logits(inp.x, inp.W)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(L.astype(np.float32)))
    assert np.array_equal(host_bits(outb), oracle.round_bf16(L))
    # the legacy BF16 output really loses bits on this workload
    assert np.any(oracle.bf16_bits_to_f64(host_bits(outb)) != L)


@pytest.mark.parametrize("K", workloads.INT_SWEEP_K)
def test_logits_integer_sweep_v32768(K):
    """The pages' integer sweep: 16 x K activations, 32,768 x K weights,
    K = 512 ... 16384; every raw FP32 output word equals the oracle's exact
    value (no tolerance), and every BF16 output word is its nearest-even
    rounding."""
    inp = workloads.integer_gemm(16, K, 32768, seed=workloads.SEED, with_targets=False)
    _say(f"int sweep K={K}")
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    out = lmh.lmhead_logits(x, W, out_dtype="fp32")
    outb = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    L, _ = oracle.logits(inp.x, inp.W, with_abs=False)
    assert L.shape == (16, 32768)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(L.astype(np.float32)))
    assert np.array_equal(host_bits(outb), oracle.round_bf16(L))


def _up(v, m):
    return (v + m - 1) // m * m


@pytest.mark.parametrize("M,K,V,pad", [
    (1, 8, 1, 0), (3, 24, 5, 8), (17, 72, 65, 0), (33, 200, 130, 16), (130, 64, 257, 8),
    (64, 136, 300, 0), (257, 96, 129, 24), (31, 1000, 511, 0), (40, 8, 1000, 0),
    (7, 13, 9, 0), (19, 77, 33, 8),
    # many tokens, K a multiple of 32 up to 8192: 1, 2, 7 and 8 stages of 32
    (260, 32, 300, 0), (300, 64, 260, 8), (270, 224, 513, 0), (512, 256, 520, 8),
    # many tokens on the 64-wide-stage kernel: K not a multiple of 32, K > 8192
    (300, 200, 700, 8), (264, 8224, 300, 0),
    # up to 64 tokens with K <= 4096: 128-deep stages (rings of 4 and 3), the
    # steady loop from 5 full stages on, ragged 128-deep tails (K = 1000)
    (40, 1024, 1000, 8), (64, 1000, 4100, 0), (64, 4096, 2049, 8), (40, 4096, 300, 16),
    (33, 1000, 777, 0), (16, 4096, 3000, 8), (64, 1024, 33, 0),
    # 129 - 256 tokens: one 256-token tile column, a ring of 3 stages
    (256, 1000, 1000, 8), (200, 4096, 2049, 0), (129, 640, 300, 16), (256, 8192, 513, 8),
])
def test_logits_ragged_integer_exact(M, K, V, pad):
    """Ragged M, K, V (partial tiles on every edge, K not a multiple of the
    64-wide stage nor of 8), padded leading dimensions; padding never written.
    Covers both large-tile kernels: the 32-wide-stage ring (K a multiple of
    32, K <= 8192) at 1, 2, 7 and 8 stages, and the 64-wide-stage kernel."""
    inp = workloads.integer_gemm(M, K, V, seed=M * 1000 + K + V, with_targets=False)
    _say(f"ragged logits M={M} K={K} V={V} pad={pad}")
    x = dev_bf16(inp.x, _up(K, 8) + pad)
    W = dev_bf16(inp.W, _up(K, 8) + 2 * pad)
    out = padded_out(M, V, _up(V, 4) + pad, torch.float32)
    outb = padded_out(M, V, _up(V, 8) + pad, torch.bfloat16)
    lmh.lmhead_logits(x, W, out=out, out_dtype="fp32")
    lmh.lmhead_logits(x, W, out=outb, out_dtype="bf16")
    torch.cuda.synchronize()
    L, _ = oracle.logits(inp.x, inp.W)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(L.astype(np.float32)))
    assert np.array_equal(host_bits(outb), oracle.round_bf16(L))
    assert padding_untouched(out) and padding_untouched(outb)


@pytest.mark.parametrize("M,K,V,pad", [(1, 8192, 1, 0), (5, 8192, 33, 8), (16, 8192, 1000, 16),
                                       (9, 16384, 4097, 0), (2, 8192, 65, 24),
                                       (16, 8192, 40000, 8), (3, 8192, 131072, 0)])
def test_logits_row_group_kernel_integer_exact(M, K, V, pad):
    """The few-token kernel that streams 32 vocabulary rows at a time (M <= 16,
    K >= 8192, a multiple of 512): ragged V (a partial last row group, fewer
    than 32 rows in all), M from 1 to 16, padded leading dimensions, several
    row groups per workgroup (V = 40000, 131072); bit-exact FP32 and BF16
    logits on integers (|logit| <= 64 K < 2^24)."""
    x_bits, W_bits = workloads.integer_operands([(M, K), (V, K)], seed=23 + M + K + V)
    _say(f"logits rows M={M} K={K} V={V} pad={pad}")
    x = dev_bf16(x_bits, K + pad)
    W = dev_bf16(W_bits, K + 2 * pad)
    out = padded_out(M, V, _up(V, 4) + 4, torch.float32)
    lmh.lmhead_logits(x, W, out=out, out_dtype="fp32")
    outb = padded_out(M, V, _up(V, 8) + 8, torch.bfloat16)
    lmh.lmhead_logits(x, W, out=outb, out_dtype="bf16")
    torch.cuda.synchronize()
    L, _ = oracle.logits(x_bits, W_bits)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(L.astype(np.float32)))
    assert np.array_equal(host_bits(outb), oracle.round_bf16(L))
    assert padding_untouched(out) and padding_untouched(outb)


@pytest.mark.parametrize("M,V", [
    (5, 12),        # few tokens, 32-wide token tile
    (48, 1000),     # few tokens, 64-wide token tile, ragged vocabulary
    (300, 700),     # ring kernel, ragged both ways
    (1024, 2048),   # ring kernel, whole 256 x 256 tiles
])
def test_logits_k_zero_writes_zeros(M, V):
    """An empty contraction (K = 0) is the zero matrix: every kernel the
    routing can pick stores zeros (FP32 and BF16) and leaves the padding of
    the output rows alone."""
    _say(f"logits K=0 M={M} V={V}")
    x = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((V, 0), dtype=torch.bfloat16, device="cuda")
    out = padded_out(M, V, _padded_ld(V, 4), torch.float32)
    outb = padded_out(M, V, _padded_ld(V, 8), torch.bfloat16)
    lmh.lmhead_logits(x, W, out=out)
    lmh.lmhead_logits(x, W, out=outb, out_dtype="bf16")
    torch.cuda.synchronize()
    assert not np.any(_f32_bits(host_f32(out)))
    assert not np.any(host_bits(outb))
    assert padding_untouched(out) and padding_untouched(outb)


@pytest.mark.parametrize("M,V", [(100, 1000), (300, 700)])
def test_logits_xent_k_zero_records(M, V):
    """K = 0 with the records: the logits are all zero, so every record and
    the merged statistics are those of a row of V equal logits (the loss of
    a kept row is log V)."""
    tgt = np.arange(M, dtype=np.int32) % V
    tgt[1::5] = -100
    _say(f"logits+records K=0 M={M} V={V}")
    x = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((V, 0), dtype=torch.bfloat16, device="cuda")
    t = torch.from_numpy(tgt).cuda()
    out, part = lmh.lmhead_logits_xent(x, W, t)
    loss, st = lmh.lmhead_xent_merge(part, t, V)
    torch.cuda.synchronize()
    z = np.zeros((M, V), dtype=np.float32)
    assert not np.any(_f32_bits(host_f32(out)))
    _check_records(host_f32(part), oracle.xent_partial(z, tgt, block_cols=256), "records")
    ref = oracle.xent_fwd(z, tgt, -100)
    lh = host_f32(loss)
    keep = tgt != -100
    assert np.all(np.abs(lh[keep] - np.log(V)) <= 1e-6 * np.log(V))
    assert np.all(lh[~keep] == 0)
    assert np.all(np.abs(host_f32(st)[:, 1] - ref[:, 1]) <= 1e-5 * ref[:, 1])


@pytest.mark.parametrize("M,K", [
    (16, 64),       # 128 x 128 tiles
    (300, 700),     # ragged both ways
    (2048, 8192),   # 256 x 256 tiles
])
def test_dgrad_v_zero_writes_zeros(M, K):
    """V = 0: dX is the zero matrix for both output dtypes, through the
    unsplit, split-request and no-alloc entry points (an empty sum has no
    parts to split), padding untouched."""
    _say(f"dgrad V=0 M={M} K={K}")
    dl = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    assert lmh.lmhead_dgrad_workspace_bytes(M, K, 0, 4) == 0
    for dt, mult in ((torch.float32, 4), (torch.bfloat16, 8)):
        for call in ("unsplit", "split", "noalloc"):
            dX = padded_out(M, K, _padded_ld(K, mult), dt)
            if call == "noalloc":
                lmh.lmhead_dgrad_noalloc(dl, W, dX, splits=4)
            else:
                lmh.lmhead_dgrad(dl, W, dX=dX, splits=1 if call == "unsplit" else 4)
            torch.cuda.synchronize()
            assert not torch.any(dX != 0).item() and not torch.isnan(dX).any().item(), call
            assert padding_untouched(dX), call


@pytest.mark.parametrize("V,K", [
    (1000, 64),     # 128 x 128 tiles
    (4096, 2048),   # 256 x 128 tiles
    (32768, 1024),  # two workgroups per CU
])
def test_wgrad_m_zero(V, K):
    """M = 0: dW = 0 when storing; accumulating adds nothing and leaves dW
    as it was."""
    _say(f"wgrad M=0 V={V} K={K}")
    dl = torch.empty((0, V), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    dW = padded_out(V, K, _padded_ld(K, 4), torch.float32)
    lmh.lmhead_wgrad(dl, x, dW=dW)
    torch.cuda.synchronize()
    assert not torch.any(dW != 0).item() and not torch.isnan(dW).any().item()
    assert padding_untouched(dW)
    dW.fill_(1.5)
    lmh.lmhead_wgrad(dl, x, dW=dW, accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(dW == 1.5).item()


def test_logits_fp16_rejected():
    x = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lmh.LmheadError) as e:
        lmh.lmhead_logits(x, x, out=torch.zeros((4, 4), dtype=torch.float16, device="cuda"),
                          out_dtype="fp16")
    assert e.value.status == 1


def test_logits_lmhead_128_random_full():
    """M=128, K=4096, V=32768, x ~ N(0,1), W ~ N(0, 0.02^2): every logit
    within 1e-5 * S of the FP64 sum; BF16 output within S-bound + half ulp."""
    inp = workloads.lmhead_128()
    _say("lmhead_128 random logits")
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    out = lmh.lmhead_logits(x, W, out_dtype="fp32")
    outb = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    L, S = oracle.logits(inp.x, inp.W)
    assert_gemm_close(host_f32(out), L, S, 1e-5, "fp32 logits")
    gb = oracle.bf16_bits_to_f64(host_bits(outb))
    half_ulp = np.abs(L) * 2.0 ** -8
    assert np.all(np.abs(gb - L) <= 1e-5 * S + half_ulp + 1e-30)
    # same accumulation, rounded once: BF16 output = RNE of the FP32 output
    # (torch's CPU conversion, nearest-even)
    assert torch.equal(outb.cpu().view(torch.int16), out.cpu().to(torch.bfloat16).view(torch.int16))


def test_logits_lmhead_1024_random_sampled():
    """M=1024, K=8192, V=32768 (the benchmark's launch shape): 64 sampled
    rows x all V columns within 1e-5 * S; run twice, bitwise identical; the
    BF16 output is the nearest-even rounding of the FP32 one everywhere."""
    inp = workloads.lmhead_1024()
    _say("lmhead_1024 random logits")
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    out = lmh.lmhead_logits(x, W, out_dtype="fp32")
    out2 = lmh.lmhead_logits(x, W, out_dtype="fp32")
    outb = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(outb.cpu().view(torch.int16), out.cpu().to(torch.bfloat16).view(torch.int16))
    rows = np.unique(np.concatenate([np.arange(0, 1024, 32), [1, 255, 256, 511, 512, 767, 1022, 1023],
                                     np.random.default_rng(64).integers(0, 1024, 40)]))[:64]
    assert rows.size == 64
    L, S = oracle.logits(inp.x, inp.W, rows=rows)
    assert_gemm_close(host_f32(out)[rows], L, S, 1e-5, "fp32 logits 1024")


# ------------------------------------------------------------------ dgrad

@pytest.mark.parametrize("M,K,V", [(16, 64, 128), (33, 72, 130), (130, 256, 1000), (64, 8, 64),
                                   (5, 520, 4100), (9, 20, 37)])
def test_dgrad_integer_exact(M, K, V):
    """dX = dl . W on integers: bit-exact FP32 and BF16 outputs; ragged M, K,
    V with padded leading dimensions."""
    dl_bits, W_bits = workloads.integer_operands([(M, V), (V, K)], seed=7 + M + K + V)
    _say(f"dgrad int M={M} K={K} V={V}")
    dl, W = dev_bf16(dl_bits, _up(V, 8)), dev_bf16(W_bits, _up(K, 8))
    dx = padded_out(M, K, _up(K, 4) + 4, torch.float32)
    lmh.lmhead_dgrad(dl, W, dX=dx, dx_dtype="fp32")
    dxb = padded_out(M, K, _up(K, 8) + 8, torch.bfloat16)
    lmh.lmhead_dgrad(dl, W, dX=dxb, dx_dtype="bf16")
    torch.cuda.synchronize()
    ref, _ = oracle.dgrad(dl_bits, W_bits)
    assert np.array_equal(_f32_bits(host_f32(dx)), _f32_bits(ref.astype(np.float32)))
    assert np.array_equal(host_bits(dxb), oracle.round_bf16(ref))
    assert padding_untouched(dx) and padding_untouched(dxb)


def test_dgrad_random_sampled():
    """dX = dl . W at M=1024, K=8192, V=32768 with synthetic BF16 dl."""
    rng = np.random.default_rng(workloads.SEED + 3)
    dl_bits = workloads.normal_bf16(rng, (1024, 32768), 1e-3)
    W_bits = workloads.normal_bf16(rng, (32768, 8192), 0.02)
    _say("dgrad random 1024x8192x32768")
    dx = lmh.lmhead_dgrad(dev_bf16(dl_bits), dev_bf16(W_bits), dx_dtype="fp32")
    torch.cuda.synchronize()
    rows = np.array([0, 1, 100, 511, 512, 1000, 1023])
    ref, S = oracle.dgrad(dl_bits, W_bits, rows=rows)
    assert_gemm_close(host_f32(dx)[rows], ref, S, 1e-5, "dgrad")


@pytest.mark.parametrize("M,K,V,splits", [(16, 64, 1000, 2), (33, 72, 1000, 3), (130, 256, 4100, 4),
                                          (9, 20, 100, 4), (64, 8, 640, 16), (300, 520, 2000, 2)])
def test_dgrad_split_integer_exact(M, K, V, splits):
    """The V-split dgrad (FP32 partials in a workspace, then a reduction in
    split order): bit-exact on integers for FP32 and BF16 dX, ragged M, K, V,
    padded leading dimensions, a NaN-filled workspace (its contents on entry
    and its padding columns must not leak into dX)."""
    dl_bits, W_bits = workloads.integer_operands([(M, V), (V, K)], seed=11 + M + K + V)
    _say(f"dgrad split={splits} int M={M} K={K} V={V}")
    dl, W = dev_bf16(dl_bits, _up(V, 8) + 8), dev_bf16(W_bits, _up(K, 8) + 16)
    need = lmh.lmhead_dgrad_workspace_bytes(M, K, V, splits)
    assert need > 0
    ws = torch.full((need // 4 + 64,), float("nan"), device="cuda")
    dx = padded_out(M, K, _up(K, 4) + 4, torch.float32)
    lmh.lmhead_dgrad(dl, W, dX=dx, dx_dtype="fp32", splits=splits, workspace=ws)
    dxb = padded_out(M, K, _up(K, 8) + 8, torch.bfloat16)
    lmh.lmhead_dgrad(dl, W, dX=dxb, dx_dtype="bf16", splits=splits, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.dgrad(dl_bits, W_bits)
    assert np.array_equal(_f32_bits(host_f32(dx)), _f32_bits(ref.astype(np.float32)))
    assert np.array_equal(host_bits(dxb), oracle.round_bf16(ref))
    assert padding_untouched(dx) and padding_untouched(dxb)


def test_dgrad_split_vs_unsplit_benchmark_shape():
    """M=1024, K=8192, V=32768 (the step's dgrad): the default path splits V in
    two; it and the unsplit kernel are both within 1e-5 * S of the FP64 sum on
    sampled rows, the split path is bitwise repeatable, and its BF16 dX is the
    nearest-even rounding of its FP32 dX."""
    rng = np.random.default_rng(workloads.SEED + 5)
    dl_bits = workloads.normal_bf16(rng, (1024, 32768), 1e-3)
    W_bits = workloads.normal_bf16(rng, (32768, 8192), 0.02)
    assert lmh.lmhead_dgrad_workspace_bytes(1024, 8192, 32768) == 2 * 1024 * 8192 * 4
    dl, W = dev_bf16(dl_bits), dev_bf16(W_bits)
    _say("dgrad split vs unsplit 1024x8192x32768")
    d_split = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32")
    d_split2 = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32")
    d_one = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32", splits=1)
    d_bf = lmh.lmhead_dgrad(dl, W)
    torch.cuda.synchronize()
    assert torch.equal(d_split.view(torch.int32), d_split2.view(torch.int32))
    assert torch.equal(d_bf.cpu().view(torch.int16), d_split.cpu().to(torch.bfloat16).view(torch.int16))
    rows = np.array([0, 1, 255, 256, 700, 1023])
    ref, S = oracle.dgrad(dl_bits, W_bits, rows=rows)
    assert_gemm_close(host_f32(d_split)[rows], ref, S, 1e-5, "dgrad split")
    assert_gemm_close(host_f32(d_one)[rows], ref, S, 1e-5, "dgrad unsplit")


def test_dgrad_split_on_a_side_stream():
    """The split dgrad launched on another stream with the binding's own
    workspace (marked in use on that stream) equals the same call on the
    current stream bitwise; a raw stream handle without a workspace is refused."""
    M, K, V = 512, 8192, 16384
    assert lmh.lmhead_dgrad_workspace_bytes(M, K, V) == 4 * M * K * 4  # four parts
    rng = np.random.default_rng(workloads.SEED + 9)
    dl = dev_bf16(workloads.normal_bf16(rng, (M, V), 1e-3))
    W = dev_bf16(workloads.normal_bf16(rng, (V, K), 0.02))
    ref = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32", stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))
    with pytest.raises(ValueError):
        lmh.lmhead_dgrad(dl, W, dx_dtype="fp32", stream=side.cuda_stream)


# Leading dimension whose byte offsets within a 256-row tile pass the 32-bit
# range of buffer loads: (256 * ld + 64) * 2 >= 2^31.
HUGE_LD = (1 << 22) + 8


def test_gemm_generic_fallback_huge_leading_dims():
    """With leading dimensions of 4,194,312 elements, the logits, dgrad (split
    or not) and wgrad calls run the generic register-staged kernel: bit-exact
    on integers, against the oracle."""
    M, K, V = 5, 72, 40
    x_bits, W_bits, dl_bits = workloads.integer_operands([(M, K), (V, K), (M, V)], seed=99)
    _say("gemm generic fallback, huge ld")
    x, W = dev_bf16(x_bits, HUGE_LD), dev_bf16(W_bits, HUGE_LD)  # 42 MB and 336 MB buffers
    dl = dev_bf16(dl_bits)
    out = lmh.lmhead_logits(x, W, out_dtype="fp32")
    dx = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32", splits=1)
    dx2 = lmh.lmhead_dgrad(dl, W, dx_dtype="fp32", splits=2)
    dw = lmh.lmhead_wgrad(dl, x)
    torch.cuda.synchronize()
    L, _ = oracle.logits(x_bits, W_bits)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(L.astype(np.float32)))
    ref, _ = oracle.dgrad(dl_bits, W_bits)
    assert np.array_equal(_f32_bits(host_f32(dx)), _f32_bits(ref.astype(np.float32)))
    assert np.array_equal(_f32_bits(host_f32(dx2)), _f32_bits(ref.astype(np.float32)))
    ref, _ = oracle.wgrad(dl_bits, x_bits)
    assert np.array_equal(_f32_bits(host_f32(dw)), _f32_bits(ref.astype(np.float32)))


# ------------------------------------------------------------------ wgrad

@pytest.mark.parametrize("M,K,V", [(16, 64, 128), (33, 72, 136), (130, 256, 1000), (8, 8, 8),
                                   (300, 40, 520), (21, 20, 130)])
def test_wgrad_integer_exact_and_accumulate(M, K, V):
    """dW = dl^T . x on integers: bit-exact, then accumulate doubles it."""
    dl_bits, x_bits = workloads.integer_operands([(M, V), (M, K)], seed=11 + M + K + V)
    _say(f"wgrad int M={M} K={K} V={V}")
    dl, x = dev_bf16(dl_bits, _up(V, 8)), dev_bf16(x_bits, _up(K, 8))
    dw = padded_out(V, K, _up(K, 4) + 4, torch.float32)
    lmh.lmhead_wgrad(dl, x, dW=dw)
    torch.cuda.synchronize()
    ref, _ = oracle.wgrad(dl_bits, x_bits)
    assert np.array_equal(_f32_bits(host_f32(dw)), _f32_bits(ref.astype(np.float32)))
    assert padding_untouched(dw)
    lmh.lmhead_wgrad(dl, x, dW=dw, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(_f32_bits(host_f32(dw)), _f32_bits((2 * ref).astype(np.float32)))


def test_wgrad_pipelined_integer_exact():
    """wgrad at 96 tokens with many tiles (the two-workgroups-per-CU kernel),
    ragged in K and V (edge tiles both ways), into a NaN-filled padded dW: no
    element left unwritten, padding untouched, and bit-exact rows at both V
    edges and in between against the oracle."""
    M, K, V = 96, 4100, 16500
    dl_bits, x_bits = workloads.integer_operands([(M, V), (M, K)], seed=77)
    _say(f"wgrad pipelined int M={M} K={K} V={V}")
    dl, x = dev_bf16(dl_bits, _up(V, 8)), dev_bf16(x_bits, _up(K, 8))
    dw = padded_out(V, K, _up(K, 4) + 4, torch.float32)
    lmh.lmhead_wgrad(dl, x, dW=dw)
    torch.cuda.synchronize()
    assert not torch.isnan(dw).any().item()
    assert padding_untouched(dw)
    rows = np.concatenate([np.arange(0, 130), np.arange(8190, 8200), np.arange(16380, V)])
    ref, _ = oracle.wgrad(dl_bits, x_bits, rows=rows)
    assert np.array_equal(_f32_bits(host_f32(dw[torch.from_numpy(rows).cuda()])),
                          _f32_bits(ref.astype(np.float32)))


def test_wgrad_random_sampled():
    """dW = dl^T . x at M=1024, K=8192, V=32768 with synthetic BF16 dl."""
    rng = np.random.default_rng(workloads.SEED + 4)
    dl_bits = workloads.normal_bf16(rng, (1024, 32768), 1e-3)
    x_bits = workloads.normal_bf16(rng, (1024, 8192), 1.0)
    _say("wgrad random 1024x8192x32768")
    dw = lmh.lmhead_wgrad(dev_bf16(dl_bits), dev_bf16(x_bits))
    torch.cuda.synchronize()
    rows = np.array([0, 5, 4095, 4096, 20000, 32767])
    ref, S = oracle.wgrad(dl_bits, x_bits, rows=rows)
    assert_gemm_close(host_f32(dw)[rows], ref, S, 1e-5, "wgrad")


# The many-token logits GEMM over whole tiles (V, M multiples of 256, K of
# 128, at least 512 tiles) runs the persistent kernel: the next tile's first
# stages load while the finished tile is stored.  M=1024 K=128 (two stages
# per tile, the least) checks every output word; M=512 K=2048 V=65536
# (uneven tiles per workgroup: none here, 64 per XCD) sampled rows.  Padded
# outputs pre-filled with NaN: no word missed, padding untouched.
@pytest.mark.parametrize("M,K,V,pad", [(1024, 128, 32768, 0), (512, 2048, 65536, 64)])
def test_logits_persistent_integer_exact(M, K, V, pad):
    """pad > 0: x and W inside wider NaN-filled rows (lda = ldb = K + pad),
    which no whole tile may read."""
    inp = workloads.integer_gemm(M, K, V, seed=8100 + K, with_targets=False)
    _say(f"logits persistent int M={M} K={K} V={V} pad={pad}")
    x, W = dev_bf16(inp.x, K + pad), dev_bf16(inp.W, K + pad)
    out = padded_out(M, V, V + 8, torch.float32)
    outb = padded_out(M, V, V + 8, torch.bfloat16)
    lmh.lmhead_logits(x, W, out=out, out_dtype="fp32")
    lmh.lmhead_logits(x, W, out=outb, out_dtype="bf16")
    torch.cuda.synchronize()
    assert padding_untouched(out) and padding_untouched(outb)
    assert not torch.isnan(out).any().item()
    rows = None if K == 128 else np.unique(np.concatenate(
        [np.arange(0, 40), np.arange(M - 40, M), np.random.default_rng(K).integers(0, M, 48)]))
    L, _ = oracle.logits(inp.x, inp.W, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    assert np.array_equal(_f32_bits(host_f32(out[sel])), _f32_bits(L.astype(np.float32)))
    assert np.array_equal(host_bits(outb[sel]), oracle.round_bf16(L))


# More whole-tile shapes for both persistent GEMMs, bit-exact on integers
# (sampled rows against the oracle, NaN-padded outputs fully written):
# uneven tiles per workgroup (520 or 528 tiles), odd numbers of stage pairs,
# two stages, and a near miss (516 tiles, not a multiple of 8) that must take
# the non-persistent kernels with the same result.
@pytest.mark.parametrize("kind,M,K,V", [("logits", 1280, 256, 26624), ("logits", 2048, 1152, 16384),
                                        ("logits", 768, 640, 44032), ("wgrad", 256, 2560, 13312),
                                        ("wgrad", 640, 4096, 8448)])
def test_persistent_more_shapes_integer_exact(kind, M, K, V):
    rng = np.random.default_rng(M + K + V)
    _say(f"persistent shapes {kind} M={M} K={K} V={V}")
    if kind == "logits":
        inp = workloads.integer_gemm(M, K, V, seed=9000 + M, with_targets=False)
        out = padded_out(M, V, V + 8, torch.float32)
        lmh.lmhead_logits(dev_bf16(inp.x), dev_bf16(inp.W), out=out, out_dtype="fp32")
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 40)]))
        ref, _ = oracle.logits(inp.x, inp.W, rows=rows)
    else:
        dl_bits, x_bits = workloads.integer_operands([(M, V), (M, K)], seed=9100 + M)
        out = padded_out(V, K, K + 4, torch.float32)
        lmh.lmhead_wgrad(dev_bf16(dl_bits), dev_bf16(x_bits), dW=out)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, V - 1], rng.integers(0, V, 40)]))
        ref, _ = oracle.wgrad(dl_bits, x_bits, rows=rows)
    assert padding_untouched(out) and not torch.isnan(out).any().item()
    got = host_f32(out[torch.from_numpy(rows).cuda()])
    assert np.array_equal(_f32_bits(got), _f32_bits(ref.astype(np.float32)))


def test_persistent_repeatable_bitwise():
    """The persistent kernels count their direct loads and stores by hand
    (loads untracked by the compiler): twelve launches each of the logits GEMM
    and wgrad at M=1024 K=8192 V=32768 on random operands, interleaved with
    other work that changes the memory system's timing (the CE on the same
    logits, a 256 MiB fill), must all give the first launch's output bit for
    bit."""
    rng = np.random.default_rng(workloads.SEED + 91)
    x_bits = workloads.normal_bf16(rng, (1024, 8192), 1.0)
    W_bits = workloads.normal_bf16(rng, (32768, 8192), 0.02)
    dl_bits = workloads.normal_bf16(rng, (1024, 32768), 1e-3)
    x, W, dl = dev_bf16(x_bits), dev_bf16(W_bits), dev_bf16(dl_bits)
    t = torch.from_numpy(rng.integers(0, 32768, 1024).astype(np.int32)).cuda()
    _say("persistent repeatability 1024x8192x32768")
    z0 = lmh.lmhead_logits(x, W, out_dtype="fp32")
    w0 = lmh.lmhead_wgrad(dl, x)
    z = torch.empty_like(z0)
    w = torch.empty_like(w0)
    junk = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    bad = 0
    for i in range(12):
        if i % 3 == 1:
            junk.fill_(i)
        lmh.lmhead_logits(x, W, out=z, out_dtype="fp32")
        if i % 3 == 2:
            lmh.lmhead_xent_fwd(z, t)
        lmh.lmhead_wgrad(dl, x, dW=w)
        bad += int(not torch.equal(z.view(torch.int32), z0.view(torch.int32)))
        bad += int(not torch.equal(w.view(torch.int32), w0.view(torch.int32)))
    torch.cuda.synchronize()
    assert bad == 0
    rows = np.array([0, 511, 1023])
    ref, S = oracle.logits(x_bits, W_bits, rows=rows)
    assert_gemm_close(host_f32(z0)[rows], ref, S, 1e-5, "logits")


# wgrad over whole tiles with the store epilogue runs the persistent kernel:
# one workgroup per CU walking its XCD's tiles, the next tile's first two
# stages loaded while the finished tile is stored.  Cases: two stages (the
# least, M=128), three stage pairs (M=384), uneven tiles per workgroup (520
# tiles: 65 per XCD over 32 workgroups), a padded dW pre-filled with NaN, and
# operands inside wider NaN-filled rows.
@pytest.mark.parametrize("M,K,V,pad", [(128, 2048, 16640, 0), (384, 4096, 8192, 24)])
def test_wgrad_persistent_integer_exact(M, K, V, pad):
    dl_bits, x_bits = workloads.integer_operands([(M, V), (M, K)], seed=7000 + M)
    _say(f"wgrad persistent int M={M} K={K} V={V} pad={pad}")
    dl, x = dev_bf16(dl_bits, V + pad), dev_bf16(x_bits, K + pad)
    dw = padded_out(V, K, K + 4, torch.float32)
    lmh.lmhead_wgrad(dl, x, dW=dw)
    torch.cuda.synchronize()
    assert not torch.isnan(dw).any().item()
    assert padding_untouched(dw)
    if M == 128:
        ref, _ = oracle.wgrad(dl_bits, x_bits)          # every element
        assert np.array_equal(_f32_bits(host_f32(dw)), _f32_bits(ref.astype(np.float32)))
    else:
        rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(V - 300, V),
                                         np.random.default_rng(M).integers(0, V, 200)]))
        ref, _ = oracle.wgrad(dl_bits, x_bits, rows=rows)
        got = host_f32(dw[torch.from_numpy(rows).cuda()])
        assert np.array_equal(_f32_bits(got), _f32_bits(ref.astype(np.float32)))


def test_wgrad_persistent_matches_accumulate_path():
    """Random BF16 operands at M=1024 K=8192 V=32768: the store path (the
    persistent kernel) and accumulation into zeros (gemm_big's 256 x 256
    tile) sum in the same order, so dW agrees bitwise everywhere; sampled
    rows against the oracle."""
    rng = np.random.default_rng(workloads.SEED + 71)
    dl_bits = workloads.normal_bf16(rng, (1024, 32768), 1e-3)
    x_bits = workloads.normal_bf16(rng, (1024, 8192), 1.0)
    _say("wgrad persistent vs accumulate 1024x8192x32768")
    dl, x = dev_bf16(dl_bits), dev_bf16(x_bits)
    dw = lmh.lmhead_wgrad(dl, x)
    dz = torch.zeros_like(dw)
    lmh.lmhead_wgrad(dl, x, dW=dz, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dz.view(torch.int32))
    rows = np.array([0, 255, 256, 8191, 16384, 32767])
    ref, S = oracle.wgrad(dl_bits, x_bits, rows=rows)
    assert_gemm_close(host_f32(dw)[rows], ref, S, 1e-5, "wgrad")


# ------------------------------------------- steady-state paths, integer exact

def test_logits_integer_exact_interior_tiles():
    """M=512 K=1024 V=2048: 256x256 8-wave tiles, all interior, 16 full
    stages (the direct-to-LDS steady loop) -- bit-exact FP32 and BF16."""
    inp = workloads.integer_gemm(512, 1024, 2048, seed=31, with_targets=False)
    _say("logits int interior 512x1024x2048")
    x, W = dev_bf16(inp.x), dev_bf16(inp.W)
    out = lmh.lmhead_logits(x, W, out_dtype="fp32")
    outb = lmh.lmhead_logits(x, W, out_dtype="bf16")
    torch.cuda.synchronize()
    L, _ = oracle.logits(inp.x, inp.W)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(L.astype(np.float32)))
    assert np.array_equal(host_bits(outb), oracle.round_bf16(L))


def test_dgrad_integer_exact_interior_tiles():
    """M=1024 K=8192 V=4096: dgrad with its default V split in two (256x256
    8-wave tiles, FP32 partials reduced in order), the p-major W operand read
    through transposing LDS loads; sampled rows bit-exact."""
    dl_bits, W_bits = workloads.integer_operands([(1024, 4096), (4096, 8192)], seed=41)
    _say("dgrad int interior 1024x8192x4096")
    dX = lmh.lmhead_dgrad(dev_bf16(dl_bits), dev_bf16(W_bits), dx_dtype="fp32")
    torch.cuda.synchronize()
    rows = np.array([0, 3, 255, 256, 700, 1023])
    ref, _ = oracle.dgrad(dl_bits, W_bits, rows=rows)
    assert np.array_equal(_f32_bits(host_f32(dX)[rows]), _f32_bits(ref.astype(np.float32)))


def test_wgrad_integer_exact_interior_tiles():
    """M=2048 K=4096 V=8192: wgrad's 256x256 8-wave tiles (the persistent
    kernel; accumulate runs gemm_big) with both p-major operands read through
    transposing LDS loads; sampled rows bit-exact, then accumulate."""
    dl_bits, x_bits = workloads.integer_operands([(2048, 8192), (2048, 4096)], seed=43)
    _say("wgrad int interior 2048x4096x8192")
    dl, x = dev_bf16(dl_bits), dev_bf16(x_bits)
    dW = lmh.lmhead_wgrad(dl, x)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 4097, 8191])
    ref, _ = oracle.wgrad(dl_bits, x_bits, rows=rows)
    assert np.array_equal(_f32_bits(host_f32(dW)[rows]), _f32_bits(ref.astype(np.float32)))
    lmh.lmhead_wgrad(dl, x, dW=dW, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(_f32_bits(host_f32(dW)[rows]), _f32_bits((2 * ref).astype(np.float32)))


# ------------------------------------- logits + cross-entropy block records

def _check_records(p_gpu, p_ref, what):
    """m_b, X_b bit-exact; own_b exact; d_b within 1e-5 relative."""
    assert np.array_equal(_f32_bits(p_gpu[..., 0]), _f32_bits(p_ref[..., 0].astype(np.float32))), what + " m"
    assert np.array_equal(_f32_bits(p_gpu[..., 2]), _f32_bits(p_ref[..., 2].astype(np.float32))), what + " X"
    assert np.array_equal(p_gpu[..., 3], p_ref[..., 3].astype(np.float32)), what + " own"
    assert np.all(np.abs(p_gpu[..., 1] - p_ref[..., 1]) <= 1e-5 * p_ref[..., 1]), what + " d"


@pytest.mark.parametrize("M,K,V", [
    (260, 64, 1000),     # ring kernel, ragged vocabulary (last block 232 columns), 2 stages
    (512, 256, 2048),    # ring kernel, interior tiles
    (300, 200, 700),     # 64-wide-stage kernel (K not a multiple of 32)
    (264, 8224, 300),    # 64-wide-stage kernel (K > 8192)
    (100, 64, 1000),     # few tokens: records from the stored logits
    (16, 512, 1024),
])
def test_logits_xent_records_integer_exact(M, K, V):
    """Integer operands make the FP32 logits exact, so the records computed in
    the GEMM epilogue (or from the stored logits) can be held to the oracle's
    records of the exact logits; targets hit the first, last and ragged-block
    columns, some rows are ignored; the merged statistics equal the oracle's
    full-row statistics and the one-pass forward's m and X bitwise."""
    inp = workloads.integer_gemm(M, K, V, seed=M + K + V)
    tgt = inp.target.copy()
    tgt[0], tgt[1], tgt[2] = 0, V - 1, ((V - 1) // 256) * 256
    tgt[3::7] = -100
    _say(f"logits+records M={M} K={K} V={V}")
    x, W, t = dev_bf16(inp.x), dev_bf16(inp.W), torch.from_numpy(tgt).cuda()
    out, part = lmh.lmhead_logits_xent(x, W, t)
    loss, st = lmh.lmhead_xent_merge(part, t, V)
    _, st1 = lmh.lmhead_xent_fwd(out, t)
    torch.cuda.synchronize()
    L, _ = oracle.logits(inp.x, inp.W)
    z = L.astype(np.float32)
    assert np.array_equal(_f32_bits(host_f32(out)), _f32_bits(z))
    _check_records(host_f32(part), oracle.xent_partial(z, tgt, block_cols=256), "records")
    ref = oracle.xent_fwd(z, tgt, -100)
    sh, s1 = host_f32(st), host_f32(st1)
    assert np.array_equal(_f32_bits(sh[:, 0]), _f32_bits(ref[:, 0].astype(np.float32)))
    assert np.array_equal(_f32_bits(sh[:, 2]), _f32_bits(ref[:, 2].astype(np.float32)))
    assert np.array_equal(_f32_bits(sh[:, 0]), _f32_bits(s1[:, 0]))
    assert np.all(np.abs(sh[:, 1] - ref[:, 1]) <= 1e-5 * ref[:, 1])


def test_logits_xent_records_benchmark_shape():
    """M=1024 K=8192 V=32768 normal operands (the benchmark's launch shape):
    the epilogue's records merged equal the one-pass forward over the stored
    logits (m, X bitwise; d within 1e-5); sampled rows' loss against the
    oracle within the logits' own error bound; two runs bitwise equal."""
    inp = workloads.lmhead_1024()
    _say("logits+records 1024x8192x32768")
    x, W, t = dev_bf16(inp.x), dev_bf16(inp.W), torch.from_numpy(inp.target).cuda()
    out, part = lmh.lmhead_logits_xent(x, W, t)
    out2, part2 = lmh.lmhead_logits_xent(x, W, t)
    loss, st = lmh.lmhead_xent_merge(part, t, 32768)
    _, st1 = lmh.lmhead_xent_fwd(out, t)
    torch.cuda.synchronize()
    assert torch.equal(part.view(torch.int32), part2.view(torch.int32))
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    sh, s1 = host_f32(st), host_f32(st1)
    assert np.array_equal(_f32_bits(sh[:, 0]), _f32_bits(s1[:, 0]))
    assert np.array_equal(_f32_bits(sh[:, 2]), _f32_bits(s1[:, 2]))
    assert np.all(np.abs(sh[:, 1] - s1[:, 1]) <= 1e-5 * s1[:, 1])
    rows = np.array([0, 1, 511, 1023])
    L, S = oracle.logits(inp.x, inp.W, rows=rows)
    ref = oracle.xent_fwd(L.astype(np.float32), inp.target[rows], -100)
    # loss error <= 2 x (max logit error) + FP32 rounding of the statistics
    bound = 2e-5 * S.max(axis=1) + 1e-5 * np.abs(ref[:, 3]) + 1e-6
    assert np.all(np.abs(host_f32(loss)[rows] - ref[:, 3]) <= bound)


# wgrad with few tokens and many tiles runs two workgroups per CU (256 x 128
# tiles, one 64-deep LDS stage).  Integer operands make every dW entry exact,
# so the check is bit-exact: ragged K (tile rows), ragged V (tile columns),
# ragged and full token counts, padded leading dimensions, store and
# accumulate.  Sampled rows of dW include the first and the ragged last ones.
@pytest.mark.parametrize("M,K,V,pad", [(100, 2056, 8200, 0), (512, 2048, 8192, 8), (1, 2304, 8328, 0),
                                       (250, 2120, 8208, 16)])
def test_wgrad_two_per_cu_integer_exact(M, K, V, pad):
    xb, gb, wb = workloads.integer_operands([(M, K), (M, V), (V, K)], seed=5151 + M)
    x = dev_bf16(xb, K + pad)
    g = dev_bf16(gb, V + pad)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(V - 40, V),
                                     np.random.default_rng(M).integers(0, V, 64)]))
    dW = lmh.lmhead_wgrad(g, x)
    torch.cuda.synchronize()
    ref, _ = oracle.wgrad(gb, xb, rows=rows)
    assert np.array_equal(host_f32(dW).astype(np.float64)[rows], ref)
    # accumulate into an existing dW (integer start values): D += tile
    W0 = oracle.bf16_bits_to_f64(wb).astype(np.float32)
    acc = dev_f32(W0)
    lmh.lmhead_wgrad(g, x, dW=acc, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(acc).astype(np.float64)[rows], ref + W0.astype(np.float64)[rows])
