"""Host-side tests of the C-ABI boundary (no GPU needed).

Every invalid-argument path of include/lmhead.h is validated on the host
before any HIP call, so these calls return their LMH_ERR_* code without a
GPU.  Pointers below are fake addresses: no call here reaches a kernel."""
import ctypes
import os
import re

import pytest

import lm_head_fp32_amd as lmh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead.h")

OK, DTYPE, SHAPE, NULL, ALIGN, ALIAS = 0, 1, 2, 3, 4, 5
BF16, FP32, FP16 = lmh.LMH_BF16, lmh.LMH_FP32, lmh.LMH_FP16

A = 0x10000000      # fake, 16-byte aligned device addresses far apart
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lmh.library_path()):
        pytest.skip("liblmhead.so not built")
    return lmh.lib()


def _declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(lmhead_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_symbols() == sorted(lmh._SIGNATURES)


def test_python_functions_carry_the_c_names():
    """Each C entry point that computes has a Python function of the same
    name, exported by the package (the dgrad workspace form is reached
    through lmhead_dgrad's `workspace` argument)."""
    wrapped = set(_declared_symbols()) - {"lmhead_dgrad_ws"}
    for name in wrapped:
        assert callable(getattr(lmh, name, None)), name
        assert name in lmh.__all__, name


def test_library_exports_every_declared_symbol(L):
    for name in _declared_symbols():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version_and_status_strings(L):
    assert lmh.lmhead_version() == 104
    assert lmh.lmhead_status_str(0) == "LMH_OK"
    for s in range(1, 8):
        assert lmh.lmhead_status_str(s).startswith("LMH_ERR_")
    assert "unknown" in lmh.lmhead_status_str(99)


def test_logits_validation(L):
    f = L.lmhead_logits
    # fp16 output is rejected, as is an unknown dtype (the pages' option accepts
    # bf16 and fp32 only)
    assert f(A, 64, B, 64, C, 128, FP16, 16, 64, 128, None) == DTYPE
    assert f(A, 64, B, 64, C, 128, 7, 16, 64, 128, None) == DTYPE
    assert f(A, 64, B, 64, C, 128, FP32, -1, 64, 128, None) == SHAPE
    assert f(A, 64, B, 64, C, 120, FP32, 16, 64, 128, None) == SHAPE   # ldo < V
    assert f(A, 56, B, 64, C, 128, FP32, 16, 64, 128, None) == SHAPE   # ldx < K
    assert f(None, 64, B, 64, C, 128, FP32, 16, 64, 128, None) == NULL
    assert f(A, 64, None, 64, C, 128, FP32, 16, 64, 128, None) == NULL
    assert f(A, 64, B, 64, None, 128, FP32, 16, 64, 128, None) == NULL
    assert f(A + 2, 64, B, 64, C, 128, FP32, 16, 64, 128, None) == ALIGN
    assert f(A, 68, B, 64, C, 128, FP32, 16, 64, 128, None) == ALIGN    # bf16 ld % 8
    assert f(A, 64, B, 64, C, 130, FP32, 16, 64, 130, None) == ALIGN    # fp32 ld % 4
    assert f(A, 64, B, 64, C, 132, BF16, 16, 64, 132, None) == ALIGN    # bf16 out ld % 8
    assert f(A, 64, B, 64, A + 64, 128, FP32, 16, 64, 128, None) == ALIAS
    assert f(A, 64, B, 64, B, 128, FP32, 16, 64, 128, None) == ALIAS
    # empty outputs are no-ops that touch nothing
    assert f(None, 64, None, 64, None, 128, FP32, 0, 64, 128, None) == OK
    assert f(None, 64, None, 64, None, 128, FP32, 16, 64, 0, None) == OK


def test_logits_xent_validation(L):
    f = L.lmhead_logits_xent
    # (x, ldx, W, ldw, out, ldo, M, K, V, target, ignore, part, part_stride, stream)
    assert f(A, 64, B, 64, C, 1024, -1, 64, 1024, D, -100, E, 4 * 300, None) == SHAPE
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, E, 4 * 299, None) == SHAPE   # stride
    assert f(A, 64, B, 64, C, 1026, 300, 64, 1024, D, -100, E, 4 * 300, None) == ALIGN   # ldo % 4
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, E, 4 * 300 + 2, None) == ALIGN
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, E + 8, 4 * 300, None) == ALIGN
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D + 2, -100, E, 4 * 300, None) == ALIGN
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, None, -100, E, 4 * 300, None) == NULL
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, None, 4 * 300, None) == NULL
    assert f(None, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, E, 4 * 300, None) == NULL
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, C + 4096, 4 * 300, None) == ALIAS
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, C, -100, E, 4 * 300, None) == ALIAS
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, A, 4 * 300, None) == ALIAS  # part in x
    assert f(A, 64, B, 64, A, 1024, 300, 64, 1024, D, -100, E, 4 * 300, None) == ALIAS  # out over x
    # last of 4 records blocks (V = 1024, stride 1200) ends at E + (3*1200 + 1200)*4
    assert f(A, 64, B, 64, C, 1024, 300, 64, 1024, E + 4 * 3600, -100, E, 1200, None) == ALIAS
    assert f(None, 64, None, 64, None, 1024, 0, 64, 1024, None, -100, None, 0, None) == OK


def test_xent_fwd_validation(L):
    f = L.lmhead_xent_fwd
    assert f(A, 1024, -1, 1024, B, -100, C, D, None) == SHAPE
    assert f(A, 1024, 8, 0, B, -100, C, D, None) == SHAPE
    assert f(A, 1000, 8, 1024, B, -100, C, D, None) == SHAPE          # ld < n_cols
    assert f(A, 1026, 8, 1024, B, -100, C, D, None) == ALIGN          # ld % 4
    assert f(A + 4, 1024, 8, 1024, B, -100, C, D, None) == ALIGN
    assert f(A, 1024, 8, 1024, B, -100, C, D + 4, None) == ALIGN      # stats 16-B
    assert f(A, 1024, 8, 1024, B + 2, -100, C, D, None) == ALIGN      # target 4-B
    assert f(None, 1024, 8, 1024, B, -100, C, D, None) == NULL
    assert f(A, 1024, 8, 1024, None, -100, C, D, None) == NULL
    assert f(A, 1024, 8, 1024, B, -100, C, None, None) == NULL
    assert f(A, 1024, 8, 1024, B, -100, C, A + 256, None) == ALIAS    # stats over logits
    assert f(A, 1024, 8, 1024, B, -100, A, D, None) == ALIAS          # loss over logits
    assert f(A, 1024, 8, 1024, B, -100, D + 16, D, None) == ALIAS     # loss over stats
    assert f(None, 1024, 0, 1024, None, -100, None, None, None) == OK


def test_xent_partial_validation(L):
    f = L.lmhead_xent_partial
    # (logits, ld, n_rows, n_cols, col0, block_cols, target, ignore, part, part_stride, stream)
    assert f(A, 1024, -1, 1024, 0, 256, B, -100, C, 32, None) == SHAPE
    assert f(A, 1024, 8, 0, 0, 256, B, -100, C, 32, None) == SHAPE
    assert f(A, 1024, 8, 1024, -1, 256, B, -100, C, 32, None) == SHAPE      # col0 < 0
    assert f(A, 1024, 8, 1024, 0, 0, B, -100, C, 32, None) == SHAPE         # block_cols 0
    assert f(A, 1024, 8, 1024, 0, 6, B, -100, C, 32, None) == SHAPE         # not a multiple of 4
    assert f(A, 1024, 8, 1024, 0, 256, B, -100, C, 28, None) == SHAPE       # stride < 4 n
    assert f(A, 1024, 8, 1024, 0, 256, B, -100, C, 34, None) == ALIGN       # stride % 4
    assert f(A, 1024, 8, 1024, 0, 256, B, -100, C + 4, 32, None) == ALIGN   # part 16-B
    assert f(A, 1024, 8, 1024, 0, 256, B + 2, -100, C, 32, None) == ALIGN   # target 4-B
    assert f(A, 1026, 8, 1024, 0, 256, B, -100, C, 32, None) == ALIGN       # ld % 4
    assert f(None, 1024, 8, 1024, 0, 256, B, -100, C, 32, None) == NULL
    assert f(A, 1024, 8, 1024, 0, 256, None, -100, C, 32, None) == NULL
    assert f(A, 1024, 8, 1024, 0, 256, B, -100, None, 32, None) == NULL
    assert f(A, 1024, 8, 1024, 0, 256, B, -100, A + 4096, 32, None) == ALIAS  # part in logits
    assert f(A, 1024, 8, 1024, 0, 256, C, -100, C, 32, None) == ALIAS       # part over target
    # the last of 4 parts (stride 64) reaches C + 3*64*4 + 32*4: a target there aliases
    assert f(A, 1024, 8, 1024, 0, 256, C + 3 * 64 * 4, -100, C, 64, None) == ALIAS
    # n_blocks * n_rows beyond INT32_MAX
    assert f(A, 2**30, 2**20, 2**30, 0, 4, B, -100, C, 4 * 2**20, None) == SHAPE
    assert f(None, 1024, 0, 1024, 0, 256, None, -100, None, 0, None) == OK


def test_xent_merge_validation(L):
    f = L.lmhead_xent_merge
    # (part, n_parts, part_stride, n_rows, target, ignore, vocab, loss, stats, stream)
    assert f(A, 4, 32, -1, B, -100, 1000, C, D, None) == SHAPE
    assert f(A, 0, 32, 8, B, -100, 1000, C, D, None) == SHAPE               # no parts
    assert f(A, 4, 32, 8, B, -100, 0, C, D, None) == SHAPE                  # vocab 0
    assert f(A, 4, 28, 8, B, -100, 1000, C, D, None) == SHAPE               # stride < 4 n
    assert f(A, 4, 34, 8, B, -100, 1000, C, D, None) == ALIGN
    assert f(A + 8, 4, 32, 8, B, -100, 1000, C, D, None) == ALIGN
    assert f(A, 4, 32, 8, B, -100, 1000, C, D + 4, None) == ALIGN           # stats 16-B
    assert f(A, 4, 32, 8, B, -100, 1000, C + 2, D, None) == ALIGN           # loss 4-B
    assert f(None, 4, 32, 8, B, -100, 1000, C, D, None) == NULL
    assert f(A, 4, 32, 8, None, -100, 1000, C, D, None) == NULL
    assert f(A, 4, 32, 8, B, -100, 1000, C, None, None) == NULL
    assert f(A, 4, 32, 8, B, -100, 1000, C, A + 256, None) == ALIAS         # stats in parts
    assert f(A, 4, 32, 8, B, -100, 1000, A + 64, D, None) == ALIAS          # loss in parts
    assert f(A, 4, 32, 8, B, -100, 1000, D + 16, D, None) == ALIAS          # loss over stats
    assert f(None, 4, 32, 0, None, -100, 1000, None, None, None) == OK


def test_xent_bwd_validation(L):
    f = L.lmhead_xent_bwd
    args = dict(logits=A, ld=1024, stats=B, target=C, ign=-100, dloss=D, ds=0,
                g=E, ldg=1024, dt=FP32, n=8, V=1024)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["logits"], a["ld"], a["stats"], a["target"], a["ign"], a["dloss"], a["ds"],
                 a["g"], a["ldg"], a["dt"], a["n"], a["V"], None)

    assert call(dt=FP16) == DTYPE
    assert call(ds=2) == SHAPE
    assert call(ds=-1) == SHAPE
    assert call(n=-1) == SHAPE
    assert call(V=0) == SHAPE
    assert call(stats=None) == NULL
    assert call(dloss=None) == NULL
    assert call(g=None) == NULL
    assert call(stats=B + 8) == ALIGN
    assert call(ldg=1028, dt=BF16) == ALIGN
    assert call(g=A, ldg=1024, dt=BF16) == ALIAS        # bf16 in place is rejected
    assert call(g=A, ldg=2048, ld=1024) == ALIAS        # in place needs the same ld
    assert call(g=A + 64) == ALIAS                      # partial overlap
    assert call(g=B - 64) == ALIAS                      # gradient over the stats
    assert call(n=0) == OK


def test_mean_validation(L):
    f = L.lmhead_xent_mean
    assert f(A, B, -100, -1, C, D, None) == SHAPE
    assert f(None, B, -100, 8, C, D, None) == NULL
    assert f(A + 2, B, -100, 8, C, D, None) == ALIGN
    assert f(A, B, -100, 8, None, None, None) == OK       # nothing requested
    assert f(None, None, -100, 8, None, D, None) == NULL  # the target is always needed
    # loss may be NULL only when the mean itself is not requested (1/n_valid
    # depends on the targets alone); that call reaches a kernel, so only its
    # rejection with a mean output is checked here
    assert f(None, B, -100, 8, C, D, None) == NULL


def test_xent_fused_validation(L):
    f = L.lmhead_xent_fused
    # (logits, ld, n, V, target, ignore, dloss, dloss_stride, loss, stats, dlogits, ldg, dtype, s)
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, A + 2**20, 1024, FP16, None) == DTYPE
    assert f(A, 1024, -1, 1024, B, -100, C, 0, D, E, A + 2**20, 1024, FP32, None) == SHAPE
    assert f(A, 1024, 8, 0, B, -100, C, 0, D, E, A + 2**20, 1024, FP32, None) == SHAPE
    assert f(A, 1024, 8, 1024, B, -100, C, 2, D, E, A + 2**20, 1024, FP32, None) == SHAPE
    assert f(A, 1000, 8, 1024, B, -100, C, 0, D, E, A + 2**20, 1024, FP32, None) == SHAPE
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, A + 2**20, 1020, FP32, None) == SHAPE
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, A + 2**20, 1028, BF16, None) == ALIGN
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E + 4, A + 2**20, 1024, FP32, None) == ALIGN
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D + 2, E, A + 2**20, 1024, FP32, None) == ALIGN
    assert f(A, 1024, 8, 1024, None, -100, C, 0, D, E, A + 2**20, 1024, FP32, None) == NULL
    assert f(A, 1024, 8, 1024, B, -100, None, 0, D, E, A + 2**20, 1024, FP32, None) == NULL
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, None, A + 2**20, 1024, FP32, None) == NULL
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, None, 1024, FP32, None) == NULL
    # in place only as FP32 with the same leading dimension
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, A, 1024, BF16, None) == ALIAS
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, A + 64, 1024, FP32, None) == ALIAS
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, A + 4096, A + 2**20, 1024, FP32, None) == ALIAS
    assert f(A, 1024, 8, 1024, B, -100, C, 0, A, E, A + 2**20, 1024, FP32, None) == ALIAS
    assert f(A, 1024, 8, 1024, B, -100, C, 0, E + 16, E, A + 2**20, 1024, FP32, None) == ALIAS
    assert f(A, 1024, 8, 1024, B, -100, C, 0, D, E, B, 1024, FP32, None) == ALIAS
    assert f(A, 1024, 8, 1024, B, -100, A + 2**20 + 8, 0, D, E, A + 2**20, 1024, FP32, None) == ALIAS
    assert f(None, 1024, 0, 1024, None, -100, None, 0, None, None, None, 1024, FP32, None) == OK


def test_dgrad_wgrad_validation(L):
    g = L.lmhead_dgrad
    assert g(A, 128, B, 64, C, 64, FP16, 16, 64, 128, None) == DTYPE
    assert g(A, 120, B, 64, C, 64, BF16, 16, 64, 128, None) == SHAPE   # ldd < V
    assert g(A, 128, B, 64, C, 60, FP32, 16, 64, 128, None) == SHAPE   # ldx < K
    assert g(A, 128, B, 64, A, 64, BF16, 16, 64, 128, None) == ALIAS
    assert g(A + 8, 128, B, 64, C, 64, BF16, 16, 64, 128, None) == ALIGN
    assert g(None, 128, B, 64, C, 64, BF16, 16, 64, 128, None) == NULL
    w = L.lmhead_wgrad
    assert w(A, 128, B, 64, C, 60, 0, 16, 64, 128, None) == SHAPE       # ldw < K
    assert w(A, 128, B, 64, C, 66, 0, 16, 64, 128, None) == ALIGN       # fp32 ld % 4
    assert w(A, 128, B, 64, B, 64, 0, 16, 64, 128, None) == ALIAS
    assert w(None, 128, B, 64, C, 64, 0, 16, 64, 128, None) == NULL
    assert w(None, 128, None, 64, C, 64, 1, 0, 64, 128, None) == OK     # M = 0, accumulate


def test_dgrad_workspace_and_split_validation(L):
    wb = L.lmhead_dgrad_workspace_bytes
    assert wb(1024, 8192, 32768, 0) == 2 * 1024 * 8192 * 4     # default: two parts
    assert wb(4096, 16384, 131072, 0) == 0                    # enough tiles: unsplit
    assert wb(16, 64, 128, 0) == 0
    assert wb(16, 64, 128, 1) == 0
    assert wb(16, 66, 1000, 3) == 3 * 16 * 68 * 4             # K rounded up to 4
    assert wb(16, 64, 100, 4) == 2 * 16 * 64 * 4              # 64-deep parts: only two
    assert wb(-1, 64, 128, 0) == -SHAPE and wb(16, 64, 128, 17) == -SHAPE
    f = L.lmhead_dgrad_ws
    need = wb(16, 64, 1000, 2)
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, None, need, None) == NULL
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, D + 4, need, None) == ALIGN
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, D, need - 16, None) == SHAPE
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, C, need, None) == ALIAS   # on dX
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, A + 64, need, None) == ALIAS
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, -1, D, need, None) == SHAPE
    assert f(A, 1000, B, 64, C, 64, FP16, 16, 64, 1000, 2, D, need, None) == DTYPE
    # unsplit shape: the call is lmhead_dgrad (its own checks), the workspace unused
    assert f(A, 120, B, 64, C, 64, BF16, 16, 64, 128, 0, None, 0, None) == SHAPE  # ldd < V


def test_gemm_grid_limits(L):
    """A GEMM whose grid would pass 2^31 work-items is refused on the host
    (LMH_ERR_SHAPE) before anything is enqueued.  The densest grid is the
    few-token kernel's, 256 work-items per 128 x 32 output tile, so the bound
    is ceil(R / 128) * ceil(C / 32) <= 2^23 for an R x C output; with the V sum
    split the parts' 256 x 128 tiles (16 parts at most) and the reduction's
    one work-item per 4 outputs bound it as well.  Operands sit at fake
    addresses far apart, so only the grid check can fail."""
    X, Y, Z, WS = 1 << 40, 1 << 42, 1 << 50, 1 << 56
    # logits M = 2^20 tokens x V = 2^22: ceil(V/128) * ceil(M/32) = 2^32 tiles
    assert L.lmhead_logits(X, 8, Y, 8, Z, 1 << 22, FP32, 1 << 20, 8, 1 << 22, None) == SHAPE
    assert L.lmhead_logits_xent(X, 8, Y, 8, Z, 1 << 22, 1 << 20, 8, 1 << 22, WS, -100,
                                WS + (1 << 30), 4 << 20, None) == SHAPE
    # wgrad dW [2^22 x 2^16]: R = K = 2^16, C = V = 2^22 -> 2^9 * 2^17 tiles
    assert L.lmhead_wgrad(X, 1 << 22, Y, 1 << 16, Z, 1 << 16, 0, 8, 1 << 16, 1 << 22,
                          None) == SHAPE
    # dgrad dX [2^20 x 2^16]: R = K = 2^16, C = M = 2^20 -> 2^9 * 2^15 tiles
    assert L.lmhead_dgrad(X, 8, Y, 1 << 16, Z, 1 << 16, FP32, 1 << 20, 1 << 16, 8,
                          None) == SHAPE
    # split dgrad M = K = 2^17 (dX 2^34 outputs): the unsplit grid would fit
    # (2^10 * 2^12 dense tiles) but 16 parts of 256 x 128 tiles do not
    need = L.lmhead_dgrad_workspace_bytes(1 << 17, 1 << 17, 1 << 13, 2)
    assert need == 2 * (1 << 34) * 4
    assert L.lmhead_dgrad_ws(X, 1 << 13, Y, 1 << 17, Z, 1 << 17, FP32, 1 << 17, 1 << 17,
                             1 << 13, 2, WS, need, None) == SHAPE


def test_dgrad_noalloc_validation(L):
    """The no-allocation dgrad checks on the host like lmhead_dgrad_ws, and
    refuses a split whose partials exceed its fixed 64 MiB array
    (LMH_ERR_SCRATCH = 7) before any HIP call."""
    f = L.lmhead_dgrad_noalloc
    SCRATCH = 7
    assert lmh.DGRAD_NOALLOC_MAX_BYTES == 64 << 20
    assert f(A, 1000, B, 64, C, 64, FP16, 16, 64, 1000, 2, None) == DTYPE
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 17, None) == SHAPE
    assert f(A, 1000, B, 64, C, 64, FP32, 16, 64, 1000, -1, None) == SHAPE
    assert f(A, 1000, B, 64, A + 64, 64, FP32, 16, 64, 1000, 2, None) == ALIAS
    assert f(A + 8, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, None) == ALIGN
    assert f(None, 1000, B, 64, C, 64, FP32, 16, 64, 1000, 2, None) == NULL
    # 4 parts of 1024 x 8192 FP32 partials: 128 MiB > 64 MiB
    assert f(A, 32768, B, 8192, C, 8192, BF16, 1024, 8192, 32768, 4, None) == SCRATCH
    # the default split of that shape fills the array exactly: not refused
    # for size (the call would run, so it is not made here)
    assert L.lmhead_dgrad_workspace_bytes(1024, 8192, 32768, 0) == 64 << 20
    # unsplit shapes are lmhead_dgrad, with its checks
    assert f(A, 120, B, 64, C, 64, BF16, 16, 64, 128, 1, None) == SHAPE      # ldd < V


def test_diag_mfma_loop_validation(L):
    f = L.lmhead_diag_mfma_loop
    for mode in (0, 1):
        assert f(-1, 4, mode, A, None) == SHAPE
        assert f(1 << 17, 4, mode, A, None) == SHAPE     # 128 * iters must stay below 2^24
        assert f(10, -1, mode, A, None) == SHAPE
        assert f(10, 65537, mode, A, None) == SHAPE
        assert f(10, 4, mode, None, None) == NULL
        assert f(10, 4, mode, A + 4, None) == ALIGN
        assert f(10, 0, mode, None, None) == OK          # no workgroups: no-op
    assert f(10, 4, 2, A, None) == SHAPE                 # operand kind outside {0, 1}
    assert f(10, 4, -1, A, None) == SHAPE


def test_binding_rejects_cpu_tensors():
    """Host tensors never reach a kernel: every tensor argument, outputs and
    the diagnostic's sink included, must be a GPU tensor."""
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        lmh.lmhead_logits(x, x)
    with pytest.raises(TypeError):
        lmh.lmhead_diag_mfma_loop(4, 1, sink=torch.zeros(256))


def test_binding_output_dtype_follows_the_tensor():
    """The binding never stores one element type into a buffer of another: a
    passed output tensor sets the type, and a conflicting explicit dtype is an
    error raised before any pointer is read.  The logits default to BF16 when
    no output is passed (FP32 logits are opted into, as with the pages' logit
    dtype option)."""
    import inspect
    import torch
    z = torch.zeros(4, 8, dtype=torch.float32)
    t = torch.zeros(4, dtype=torch.int32)
    gb = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lmh.lmhead_xent_bwd(z, z, t, z, dlogits=gb, grad_dtype="fp32")
    with pytest.raises(ValueError):
        lmh.lmhead_xent_fused(z, t, z, dlogits=gb, grad_dtype="fp32")
    with pytest.raises(ValueError):
        lmh.lmhead_xent_bwd(z, z, t, z, in_place=True, grad_dtype="bf16")
    with pytest.raises(ValueError):
        lmh.lmhead_logits(gb, gb, out=z, out_dtype="bf16")
    with pytest.raises(ValueError):
        lmh.lmhead_dgrad(gb, gb, dX=z, dx_dtype="bf16")
    assert lmh._out_code("f", None, None, "bf16") == lmh.LMH_BF16
    assert lmh._out_code("f", z, None, "bf16") == lmh.LMH_FP32
    assert lmh._out_code("f", gb, "bf16", "fp32") == lmh.LMH_BF16
    assert inspect.signature(lmh.lmhead_logits).parameters["out_dtype"].default is None
    assert "'bf16'" in lmh.lmhead_logits.__doc__


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and
    says so, before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stdout


def test_spans_past_2_44_elements_are_refused(L):
    """A leading dimension or record stride so large that the matrix would
    span more than 2^44 elements is refused on the host (LMH_ERR_SHAPE), so
    no span or kernel offset computed from it can overflow 64 bits."""
    big = 1 << 62
    f = L.lmhead_logits
    assert f(A, 64, B, 64, C, big, FP32, 16, 64, 128, None) == SHAPE          # ldo
    assert f(A, big, B, 64, C, 128, FP32, 16, 64, 128, None) == SHAPE         # ldx
    assert f(A, 64, B, (1 << 44) - 8, C, 128, FP32, 16, 64, 128, None) == SHAPE  # V rows of W
    assert f(A, 64, B, 64, C, (1 << 44) + 4, FP32, 1, 64, 128, None) == SHAPE  # ld alone too large
    g = L.lmhead_xent_fwd
    assert g(A, big, 4, 1024, B, -100, C, D, None) == SHAPE
    assert g(A, 1 << 43, 3, 1024, B, -100, C, D, None) == SHAPE                # 2 x 2^43 + 1024
    p = L.lmhead_xent_partial
    assert p(A, 1024, 8, 1024, 0, 256, B, -100, C, big, None) == SHAPE
    assert p(A, 1024, 8, 1024, 0, (1 << 63) - 4, B, -100, C, 32, None) == SHAPE   # block_cols
    m = L.lmhead_xent_merge
    assert m(A, 4, big, 8, B, -100, 1000, C, D, None) == SHAPE
    x = L.lmhead_logits_xent
    assert x(A, 64, B, 64, C, 1024, 300, 64, 1024, D, -100, E, big, None) == SHAPE

    # the dgrad workspace size for an output past 2^44 elements is refused, not overflowed
    huge = (1 << 31) - 1
    assert L.lmhead_dgrad_workspace_bytes(huge, huge, 1024, 2) == -SHAPE
    assert L.lmhead_dgrad_ws(A, 1024, B, huge, C, huge, FP32, huge, huge, 1024, 2, E, 1 << 40,
                             None) == SHAPE
    assert L.lmhead_dgrad_noalloc(A, 1024, B, huge, C, huge, FP32, huge, huge, 1024, 2,
                                  None) == SHAPE
