"""FP64 CPU oracle for the LM-head path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library never does, and this
package never imports the product: the two share nothing but the seeded input
bytes made by ``workloads``.

The arithmetic lives in ``oracle.c`` (plain C, FP64); this module only
marshals numpy arrays.  What each routine computes, with the passage of the
pages it follows:

* ``logits``  -- logits[i][j] = sum_k x[i][k] * W[j][k] with BF16 operands,
  the GEMM whose FP32 accumulator becomes the FP32 logits (Megatron-LM pull
  request "Add mixed-precision (FP32) LM output logits", section "What does
  this PR do?").  Returned in FP64 together with S = sum_k |x w|, the scale
  of the rounding-error bound.
* ``dgrad`` / ``wgrad`` -- the same plain contraction for dX = dlogits . W and
  dW = dlogits^T . x, the GEMMs that take the BF16-cast logits gradient (same
  section: the backward casts the gradient back to BF16 for the GEMMs).
* ``xent_fwd`` -- per-row {m, d, X_y, loss}: the n_rows x 4 m_d_X_y record
  kept for the backward (Transformer Engine issue "[Pytorch] change fused
  cross entropy backward grad to fp32 and reduce one read/...", discussion),
  with the row loss as its fourth column.
* ``xent_mean`` -- mean over rows whose target is not ignore_index.
* ``xent_bwd`` -- dloss * (softmax - one_hot) in FP64 (same issue, section
  "Changes": the backward gradient is computed in FP32 or better).
* ``round_bf16`` -- round to nearest BF16, ties to even (the legacy BF16
  logits and the backward's BF16 cast).

Parity pins: every routine above is checked in ``tests/test_oracle_pins.py``
against integer arithmetic, closed forms, brute force or finite differences.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# $LMH_ORACLE_LIB selects another build of oracle.c (the sanitized one).
_LIB_PATH = os.environ.get("LMH_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build(sanitize=_LIB_PATH == _build.SAN_LIB)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_gemm_bf16.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64,
                                  _i64, _vp, _i64, _i64, _vp, _vp, ctypes.c_int]
    lib.orc_gemm_bf16.restype = ctypes.c_int
    lib.orc_xent_fwd.argtypes = [_vp, _i64, _i64, _vp, _i32, _i64, _vp, _vp, ctypes.c_int]
    lib.orc_xent_fwd.restype = ctypes.c_int
    lib.orc_xent_bwd.argtypes = [_vp, _i64, _i64, _vp, _i32, _vp, _i64,
                                 _i64, _vp, _vp, ctypes.c_int]
    lib.orc_xent_bwd.restype = ctypes.c_int
    lib.orc_xent_partial.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _i64, _vp, _vp,
                                     ctypes.c_int]
    lib.orc_xent_partial.restype = ctypes.c_int
    lib.orc_xent_merge.argtypes = [_vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp]
    lib.orc_xent_merge.restype = None
    lib.orc_xent_mean.argtypes = [_vp, _vp, _i32, _i64, _vp]
    lib.orc_xent_mean.restype = ctypes.c_int
    lib.orc_round_bf16_array.argtypes = [_vp, _i64, _vp]
    lib.orc_round_bf16_array.restype = None
    lib.orc_default_threads.argtypes = []
    lib.orc_default_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses: $LMH_ORACLE_THREADS, else $OMP_NUM_THREADS,
    else every online core."""
    for var in ("LMH_ORACLE_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit() and int(v) > 0:
            return int(v)
    return int(_load().orc_default_threads())


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _rowmajor(a, dtype, name):
    """Accept a 2-D array whose rows may be padded (a column slice of a wider
    buffer); return it with its leading dimension in elements."""
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"{name}: expected {np.dtype(dtype)}, got {a.dtype}")
    if a.ndim != 2:
        raise ValueError(f"{name}: expected 2-D")
    item = a.dtype.itemsize
    if a.shape[0] > 0 and a.shape[1] > 0:
        if a.strides[1] != item or a.strides[0] % item or a.strides[0] < a.shape[1] * item:
            a = np.ascontiguousarray(a)
    ld = a.strides[0] // item if a.shape[0] > 1 else max(a.shape[1], 1)
    return a, int(ld)


def _rows_arg(rows, n):
    if rows is None:
        return None, n
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= n)):
        raise ValueError("rows out of range")
    return r, int(r.size)


def _nthreads(nthreads):
    return int(nthreads) if nthreads else default_threads()


def _gemm(a, a_si, a_sp, b, b_sj, b_sp, n_rows, rows, nj, np_, with_abs, nthreads):
    c = np.empty((n_rows, nj), dtype=np.float64)
    s = np.empty((n_rows, nj), dtype=np.float64) if with_abs else None
    rc = _load().orc_gemm_bf16(_ptr(a), a_si, a_sp, _ptr(b), b_sj, b_sp,
                               n_rows, _ptr(rows), nj, np_, _ptr(c), _ptr(s),
                               _nthreads(nthreads))
    if rc != 0:
        raise ValueError(f"orc_gemm_bf16 failed ({rc})")
    return c, s


def logits(x, W, rows=None, with_abs=True, nthreads=None):
    """L[r][v] = sum_k x[i_r][k] * W[v][k] (FP64), and S = sum_k |x w|.

    x: uint16 BF16 bits [M, K]; W: uint16 BF16 bits [V, K]; rows selects
    activation rows (default all)."""
    x, ldx = _rowmajor(x, np.uint16, "x")
    W, ldw = _rowmajor(W, np.uint16, "W")
    M, K = x.shape
    V, K2 = W.shape
    if K != K2:
        raise ValueError("x and W disagree on K")
    r, n = _rows_arg(rows, M)
    return _gemm(x, ldx, 1, W, ldw, 1, n, r, V, K, with_abs, nthreads)


def dgrad(dl, W, rows=None, with_abs=True, nthreads=None):
    """dX[r][k] = sum_v dl[i_r][v] * W[v][k] (FP64) for BF16 dl [M, V] and
    W [V, K]; rows selects rows of M."""
    dl, ldd = _rowmajor(dl, np.uint16, "dlogits")
    W, ldw = _rowmajor(W, np.uint16, "W")
    M, V = dl.shape
    V2, K = W.shape
    if V != V2:
        raise ValueError("dlogits and W disagree on V")
    r, n = _rows_arg(rows, M)
    return _gemm(dl, ldd, 1, W, 1, ldw, n, r, K, V, with_abs, nthreads)


def wgrad(dl, x, rows=None, with_abs=True, nthreads=None):
    """dW[r][k] = sum_m dl[m][i_r] * x[m][k] (FP64) for BF16 dl [M, V] and
    x [M, K]; rows selects rows of V."""
    dl, ldd = _rowmajor(dl, np.uint16, "dlogits")
    x, ldx = _rowmajor(x, np.uint16, "x")
    M, V = dl.shape
    M2, K = x.shape
    if M != M2:
        raise ValueError("dlogits and x disagree on M")
    r, n = _rows_arg(rows, V)
    return _gemm(dl, 1, ldd, x, 1, ldx, n, r, K, M, with_abs, nthreads)


def xent_fwd(z, target, ignore_index=-100, rows=None, nthreads=None):
    """stats[r] = {m, d, X_y, loss} (FP64) for FP32 logits z [n, V]."""
    z, ld = _rowmajor(z, np.float32, "logits")
    t = np.ascontiguousarray(np.asarray(target, dtype=np.int32))
    n, V = z.shape
    if t.shape != (n,):
        raise ValueError("target must be [n_rows]")
    r, nsel = _rows_arg(rows, n)
    st = np.empty((nsel, 4), dtype=np.float64)
    rc = _load().orc_xent_fwd(_ptr(z), ld, V, _ptr(t), int(ignore_index), nsel,
                              _ptr(r), _ptr(st), _nthreads(nthreads))
    if rc != 0:
        raise ValueError(f"orc_xent_fwd failed ({rc}): target out of range?")
    return st


def xent_partial(z, target, ignore_index=-100, col0=0, block_cols=4096, rows=None, nthreads=None):
    """Partial statistics of a slice of logits rows z [n, ncols] that holds
    the global columns [col0, col0 + ncols), in blocks of block_cols columns:
    an array [n_blocks, n_sel, 4] of {m_b, d_b, X_b, own_b} (FP64)."""
    z, ld = _rowmajor(z, np.float32, "logits")
    t = np.ascontiguousarray(np.asarray(target, dtype=np.int32))
    n, nc = z.shape
    if t.shape != (n,):
        raise ValueError("target must be [n_rows]")
    r, nsel = _rows_arg(rows, n)
    nb = (nc + block_cols - 1) // block_cols
    part = np.empty((nb, nsel, 4), dtype=np.float64)
    rc = _load().orc_xent_partial(_ptr(z), ld, nc, int(col0), int(block_cols), _ptr(t),
                                  int(ignore_index), nsel, _ptr(r), _ptr(part),
                                  _nthreads(nthreads))
    if rc != 0:
        raise ValueError(f"orc_xent_partial failed ({rc})")
    return part


def xent_merge(part, target, vocab, ignore_index=-100):
    """Merge partial records part [n_parts, n, 4] (FP64) into stats [n, 4] =
    {m, d, X_y, loss}; unowned or out-of-range targets give NaN X and loss."""
    p = np.ascontiguousarray(np.asarray(part, dtype=np.float64))
    t = np.ascontiguousarray(np.asarray(target, dtype=np.int32))
    if p.ndim != 3 or p.shape[2] != 4 or p.shape[1] != t.size:
        raise ValueError("part must be [n_parts, n_rows, 4]")
    st = np.empty((t.size, 4), dtype=np.float64)
    _load().orc_xent_merge(_ptr(p), p.shape[0], 4 * t.size, t.size, _ptr(t), int(ignore_index),
                           int(vocab), _ptr(st))
    return st


def xent_mean(loss, target, ignore_index=-100):
    """(mean, 1/n_valid, n_valid) over rows whose target != ignore_index."""
    lo = np.ascontiguousarray(np.asarray(loss, dtype=np.float64))
    t = np.ascontiguousarray(np.asarray(target, dtype=np.int32))
    if lo.shape != t.shape or lo.ndim != 1:
        raise ValueError("loss and target must both be [n_rows]")
    out = np.zeros(3, dtype=np.float64)
    _load().orc_xent_mean(_ptr(lo), _ptr(t), int(ignore_index), lo.size, _ptr(out))
    return float(out[0]), float(out[1]), int(out[2])


def xent_bwd(z, target, ignore_index, dloss, rows=None, nthreads=None):
    """g[r][j] = dloss_i * (softmax(z_i)_j - [j == y_i]) in FP64.

    dloss: a scalar (broadcast to every row) or an [n] array (per row)."""
    z, ld = _rowmajor(z, np.float32, "logits")
    t = np.ascontiguousarray(np.asarray(target, dtype=np.int32))
    n, V = z.shape
    if t.shape != (n,):
        raise ValueError("target must be [n_rows]")
    dl = np.asarray(dloss, dtype=np.float64)
    if dl.ndim == 0:
        dl = np.ascontiguousarray(dl.reshape(1))
        stride = 0
    else:
        if dl.shape != (n,):
            raise ValueError("per-row dloss must be [n_rows]")
        dl = np.ascontiguousarray(dl)
        stride = 1
    r, nsel = _rows_arg(rows, n)
    g = np.empty((nsel, V), dtype=np.float64)
    rc = _load().orc_xent_bwd(_ptr(z), ld, V, _ptr(t), int(ignore_index), _ptr(dl), stride,
                              nsel, _ptr(r), _ptr(g), _nthreads(nthreads))
    if rc != 0:
        raise ValueError(f"orc_xent_bwd failed ({rc}): target out of range?")
    return g


def round_bf16(values):
    """Round FP64 values to BF16 (nearest, ties to even); returns uint16 bits."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_round_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_bits_to_f64(bits):
    """Exact widening of BF16 bit patterns (the top half of a binary32 word)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
