"""lm_head_fp32_amd -- FP32 LM-head logits and fused FP32 cross-entropy on
MI355X (gfx950), as a thin Python binding over ``liblmhead.so``.

Every function here has the name of the C entry point it calls (see
``include/lmhead.h``) and only marshals arguments: checks that tensors are
on the GPU with the right dtype, reads pointers, leading dimensions and the
current stream, allocates outputs the caller did not pass, and raises
``LmheadError`` on a non-zero status.  All arithmetic runs in the HIP
kernels.  There is no fallback: without the built library every call raises.

Shapes (row-major, last dimension contiguous, rows may be padded):
  x [M, K] bf16, W [V, K] bf16 -> logits [M, V] fp32 or bf16
  logits [n, V] fp32, target [n] int32 -> loss [n] fp32, stats [n, 4] fp32
  stats {m, d, X_y, loss} per row; dlogits [n, V] fp32 or bf16
  dgrad: dlogits [M, V] bf16, W [V, K] bf16 -> dX [M, K]
  wgrad: dlogits [M, V] bf16, x [M, K] bf16 -> dW [V, K] fp32
"""
import ctypes
import os

import torch

__all__ = [
    "LMH_BF16", "LMH_FP32", "LMH_FP16", "STATS_COLS", "DGRAD_NOALLOC_MAX_BYTES", "LmheadError",
    "lib", "library_path", "lmhead_logits", "lmhead_logits_xent", "lmhead_xent_fwd",
    "lmhead_xent_partial", "lmhead_xent_merge", "lmhead_xent_mean", "lmhead_xent_bwd",
    "lmhead_xent_fused", "lmhead_dgrad", "lmhead_dgrad_noalloc", "lmhead_wgrad",
    "lmhead_status_str", "lmhead_version", "lmhead_diag_mfma_loop", "lmhead_dgrad_workspace_bytes",
]

LMH_BF16, LMH_FP32, LMH_FP16 = 0, 1, 2
STATS_COLS = 4  # {m, d, X_y, loss}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblmhead.so")
_lib = None

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p

# (name, argtypes) of every entry point in include/lmhead.h
_SIGNATURES = {
    "lmhead_status_str": ([_i32], ctypes.c_char_p),
    "lmhead_version": ([], _i32),
    "lmhead_logits": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i64, _i64, _i64, _vp], _i32),
    "lmhead_logits_xent": ([_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64,
                            _vp], _i32),
    "lmhead_xent_fwd": ([_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp], _i32),
    "lmhead_xent_partial": ([_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _vp], _i32),
    "lmhead_xent_merge": ([_vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp, _vp, _vp], _i32),
    "lmhead_xent_mean": ([_vp, _vp, _i32, _i64, _vp, _vp, _vp], _i32),
    "lmhead_xent_fused": ([_vp, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _vp, _vp, _vp, _i64, _i32,
                           _vp], _i32),
    "lmhead_xent_bwd": ([_vp, _i64, _vp, _vp, _i32, _vp, _i64, _vp, _i64, _i32, _i64, _i64,
                         _vp], _i32),
    "lmhead_dgrad": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i64, _i64, _i64, _vp], _i32),
    "lmhead_wgrad": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i64, _i64, _i64, _vp], _i32),
    "lmhead_diag_mfma_loop": ([_i64, _i64, _i32, _vp, _vp], _i32),
    "lmhead_dgrad_workspace_bytes": ([_i64, _i64, _i64, _i32], _i64),
    "lmhead_dgrad_ws": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i64, _i64, _i64, _i32, _vp, _i64,
                         _vp], _i32),
    "lmhead_dgrad_noalloc": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i64, _i64, _i64, _i32,
                              _vp], _i32),
}

DGRAD_NOALLOC_MAX_BYTES = 64 << 20  # LMH_DGRAD_NOALLOC_MAX_BYTES in lmhead.h


class LmheadError(RuntimeError):
    def __init__(self, fn, status):
        self.status = int(status)
        super().__init__(f"{fn}: {lmhead_status_str(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded ``liblmhead.so`` (ctypes) with every signature declared.
    Raises if the library has not been built -- there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
            "g.build()'` (hipcc, gfx950)")
    handle = ctypes.CDLL(_LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = res
    _lib = handle
    return handle


def lmhead_status_str(status) -> str:
    return lib().lmhead_status_str(int(status)).decode()


def lmhead_version() -> int:
    return int(lib().lmhead_version())


# ------------------------------------------------------------- marshalling

_DT = {"bf16": LMH_BF16, "fp32": LMH_FP32, "fp16": LMH_FP16,
       torch.bfloat16: LMH_BF16, torch.float32: LMH_FP32, torch.float16: LMH_FP16}
_TORCH_DT = {LMH_BF16: torch.bfloat16, LMH_FP32: torch.float32, LMH_FP16: torch.float16}


def _dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    if dt not in _DT:
        raise ValueError(f"unknown dtype {dt!r}")
    return _DT[dt]


def _out_code(fn, out, dtype_arg, default):
    """Element-type code of an output: the passed tensor's own dtype (a
    conflicting explicit dtype is an error, so that the kernel never stores
    one type into a buffer of another), else dtype_arg, else the default."""
    if out is not None:
        if not isinstance(out, torch.Tensor):
            raise TypeError(f"{fn}: the output must be a tensor")
        code = _DT.get(out.dtype)
        if code is None:
            raise TypeError(f"{fn}: unsupported output dtype {out.dtype}")
        if dtype_arg is not None and _dtype_code(dtype_arg) != code:
            raise ValueError(f"{fn}: the output tensor is {out.dtype}, not {dtype_arg!r}")
        return code
    return _dtype_code(default if dtype_arg is None else dtype_arg)


def _check(fn, status):
    if status != 0:
        raise LmheadError(fn, status)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on_current_device(t, name):
    """The kernels run on the current device (HIP launches target it), so a
    tensor on another GPU is refused rather than read from the wrong one."""
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _mat(t, name, dtype):
    """(pointer, ld) of a 2-D GPU tensor with a contiguous last dimension."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    _on_current_device(t, name)
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    ld = t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))
    return _vp(t.data_ptr()), int(ld)


def _vec(t, name, dtype, n):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    _on_current_device(t, name)
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() != n or (n > 1 and not t.is_contiguous()):
        raise ValueError(f"{name}: expected {n} contiguous elements")
    return _vp(t.data_ptr())


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _empty_rows(rows, cols, dtype, like):
    """[rows, cols] output whose leading dimension is rounded up to the
    library's alignment (4 elements for fp32, 8 for bf16); the padding
    columns are never written."""
    mult = 4 if dtype == torch.float32 else 8
    ld = max((cols + mult - 1) // mult * mult, mult)
    if ld == cols:
        return torch.empty((rows, cols), dtype=dtype, device=like.device)
    return torch.empty((rows, ld), dtype=dtype, device=like.device)[:, :cols]


# --------------------------------------------------------------- the calls

def lmhead_logits(x, W, out=None, out_dtype=None, stream=None):
    """logits[M, V] = x[M, K] . W[V, K]^T; out_dtype 'fp32' keeps the FP32
    accumulator, 'bf16' rounds it (legacy); 'fp16' is rejected.  The default
    is the output tensor's dtype when `out` is given, else 'bf16': as with
    the logit-dtype option of Megatron-LM "Add mixed-precision (FP32) LM
    output logits" (section "Tests"), FP32 logits are opted into."""
    code = _out_code("lmhead_logits", out, out_dtype, "bf16")
    px, ldx = _mat(x, "x", torch.bfloat16)
    pw, ldw = _mat(W, "W", torch.bfloat16)
    M, K = x.shape
    V = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("x and W disagree on K")
    if out is None:
        if code not in (LMH_BF16, LMH_FP32):
            _check("lmhead_logits", 1)
        out = _empty_rows(M, V, _TORCH_DT[code], x)
    po, ldo = _mat(out, "out", out.dtype)
    if out.shape != (M, V):
        raise ValueError("out must be [M, V]")
    _check("lmhead_logits", lib().lmhead_logits(px, ldx, pw, ldw, po, ldo, code, M, K, V,
                                                _stream(stream)))
    return out


LOGITS_STATS_BLOCK = 256  # vocabulary columns per record of lmhead_logits_xent


def lmhead_logits_xent(x, W, target, ignore_index=-100, out=None, part=None, stream=None):
    """FP32 logits [M, V] and their cross-entropy records part [ceil(V/256),
    M, 4] (as lmhead_xent_partial with block_cols=256), the records computed
    in the GEMM's epilogue where the kernel supports it.  Returns (out, part)."""
    px, ldx = _mat(x, "x", torch.bfloat16)
    pw, ldw = _mat(W, "W", torch.bfloat16)
    M, K = x.shape
    V = W.shape[0]
    pt = _vec(target, "target", torch.int32, M)
    if out is None:
        out = _empty_rows(M, V, torch.float32, x)
    po, ldo = _mat(out, "out", torch.float32)
    nb = max((V + LOGITS_STATS_BLOCK - 1) // LOGITS_STATS_BLOCK, 1)
    if part is None:
        part = torch.empty((nb, M, STATS_COLS), dtype=torch.float32, device=x.device)
    pp, stride = _parts(part, M)
    _check("lmhead_logits_xent", lib().lmhead_logits_xent(px, ldx, pw, ldw, po, ldo, M, K, V, pt,
                                                          int(ignore_index), pp, stride,
                                                          _stream(stream)))
    return out, part


def lmhead_xent_fwd(logits, target, ignore_index=-100, loss=None, stats=None, stream=None):
    """Fused CE forward: returns (loss [n], stats [n, 4] = {m, d, X_y, loss})."""
    pz, ld = _mat(logits, "logits", torch.float32)
    n, V = logits.shape
    pt = _vec(target, "target", torch.int32, n)
    if stats is None:
        stats = _empty((n, STATS_COLS), torch.float32, logits)
    if loss is None:
        loss = _empty((n,), torch.float32, logits)
    ps = _vec(stats, "stats", torch.float32, n * STATS_COLS)
    pl = _vec(loss, "loss", torch.float32, n) if loss is not False else None
    _check("lmhead_xent_fwd", lib().lmhead_xent_fwd(pz, ld, n, V, pt, int(ignore_index), pl, ps,
                                                    _stream(stream)))
    return (loss if loss is not False else None), stats


def lmhead_xent_partial(logits, target, ignore_index=-100, col0=0, block_cols=4096, part=None,
                        stream=None):
    """Split-vocabulary CE forward, step 1: per column block of each row,
    {m_b, d_b, X_b, own_b}.  The logits slice holds the global columns
    [col0, col0 + n_cols); targets are global.  Returns part [n_blocks,
    n_rows, 4] (any [n_blocks, n_rows, 4] FP32 view with a contiguous last
    two dimensions may be passed in)."""
    pz, ld = _mat(logits, "logits", torch.float32)
    n, nc = logits.shape
    pt = _vec(target, "target", torch.int32, n)
    nb = max((nc + block_cols - 1) // block_cols, 1) if block_cols > 0 else 1
    if part is None:
        part = torch.empty((nb, n, STATS_COLS), dtype=torch.float32, device=logits.device)
    pp, stride = _parts(part, n)
    _check("lmhead_xent_partial",
           lib().lmhead_xent_partial(pz, ld, n, nc, int(col0), int(block_cols), pt,
                                     int(ignore_index), pp, stride, _stream(stream)))
    return part


def lmhead_xent_merge(part, target, vocab, ignore_index=-100, loss=None, stats=None, stream=None):
    """Split-vocabulary CE forward, step 2: merge part [n_parts, n_rows, 4]
    into (loss [n], stats [n, 4] = {m, d, X_y, loss}), as lmhead_xent_fwd."""
    n = target.numel()
    pt = _vec(target, "target", torch.int32, n)
    pp, stride = _parts(part, n)
    if stats is None:
        stats = _empty((n, STATS_COLS), torch.float32, part)
    if loss is None:
        loss = _empty((n,), torch.float32, part)
    ps = _vec(stats, "stats", torch.float32, n * STATS_COLS)
    pl = _vec(loss, "loss", torch.float32, n) if loss is not False else None
    _check("lmhead_xent_merge",
           lib().lmhead_xent_merge(pp, part.shape[0], stride, n, pt, int(ignore_index), int(vocab),
                                   pl, ps, _stream(stream)))
    return (loss if loss is not False else None), stats


def _parts(part, n):
    """(pointer, stride between parts in elements) of an FP32 [P, n, 4] tensor."""
    if not isinstance(part, torch.Tensor) or not part.is_cuda or part.dtype != torch.float32:
        raise TypeError("part: expected a GPU float32 tensor")
    _on_current_device(part, "part")
    if part.dim() != 3 or part.shape[1] != n or part.shape[2] != STATS_COLS:
        raise ValueError(f"part: expected shape [n_parts, {n}, {STATS_COLS}]")
    if n > 0 and (part.stride(2) != 1 or part.stride(1) != STATS_COLS):
        raise ValueError("part: each part must be a contiguous [n_rows, 4] block")
    stride = part.stride(0) if part.shape[0] > 1 else STATS_COLS * n
    return _vp(part.data_ptr()), int(stride)


def lmhead_xent_mean(loss, target, ignore_index=-100, mean=None, inv_nvalid=None, stream=None):
    """Mean over non-ignored rows: returns (mean [1], inv_nvalid [1]) on the GPU.
    loss=None computes 1/n_valid only (from the targets) and returns
    (None, inv_nvalid)."""
    n = target.numel()
    pt = _vec(target, "target", torch.int32, n)
    if loss is None:
        if inv_nvalid is None:
            inv_nvalid = _empty((1,), torch.float32, target)
        pi = _vec(inv_nvalid, "inv_nvalid", torch.float32, 1)
        _check("lmhead_xent_mean", lib().lmhead_xent_mean(None, pt, int(ignore_index), n, None, pi,
                                                          _stream(stream)))
        return None, inv_nvalid
    pl = _vec(loss, "loss", torch.float32, n)
    if mean is None:
        mean = _empty((1,), torch.float32, loss)
    if inv_nvalid is None:
        inv_nvalid = _empty((1,), torch.float32, loss)
    pm = _vec(mean, "mean", torch.float32, 1)
    pi = _vec(inv_nvalid, "inv_nvalid", torch.float32, 1)
    _check("lmhead_xent_mean", lib().lmhead_xent_mean(pl, pt, int(ignore_index), n, pm, pi,
                                                      _stream(stream)))
    return mean, inv_nvalid


def lmhead_xent_bwd(logits, stats, target, dloss, ignore_index=-100, dlogits=None,
                    grad_dtype=None, in_place=False, stream=None):
    """Fused CE backward: dlogits = dloss_i * (softmax - one_hot) in FP32.

    dloss: a GPU fp32 tensor of 1 element (every row) or n elements (per row).
    grad_dtype 'fp32' or 'bf16' (default: the dtype of `dlogits` when given,
    else 'fp32'); in_place=True writes over `logits` (fp32)."""
    code = _out_code("lmhead_xent_bwd", logits if in_place else dlogits, grad_dtype, "fp32")
    pz, ld = _mat(logits, "logits", torch.float32)
    n, V = logits.shape
    ps = _vec(stats, "stats", torch.float32, n * STATS_COLS)
    pt = _vec(target, "target", torch.int32, n)
    if not isinstance(dloss, torch.Tensor) or not dloss.is_cuda or dloss.dtype != torch.float32:
        raise TypeError("dloss: expected a GPU fp32 tensor")
    _on_current_device(dloss, "dloss")
    if dloss.numel() == 1:
        stride = 0
    elif dloss.numel() == n and dloss.is_contiguous():
        stride = 1
    else:
        raise ValueError("dloss must hold 1 or n_rows contiguous values")
    pd = _vp(dloss.data_ptr())
    if in_place:
        dlogits = logits
    elif dlogits is None:
        if code not in (LMH_BF16, LMH_FP32):
            _check("lmhead_xent_bwd", 1)
        dlogits = _empty_rows(n, V, _TORCH_DT[code], logits)
    pg, ldg = _mat(dlogits, "dlogits", dlogits.dtype)
    if dlogits.shape != (n, V):
        raise ValueError("dlogits must be [n, V]")
    _check("lmhead_xent_bwd", lib().lmhead_xent_bwd(pz, ld, ps, pt, int(ignore_index), pd, stride,
                                                    pg, ldg, code, n, V, _stream(stream)))
    return dlogits


def lmhead_xent_fused(logits, target, dloss, ignore_index=-100, dlogits=None, grad_dtype=None,
                      in_place=False, loss=None, stats=None, stream=None):
    """Forward and backward in one read of the logits, for an upstream
    gradient known before the forward: returns (loss [n], stats [n, 4],
    dlogits).  dloss and grad_dtype as in lmhead_xent_bwd; in_place=True
    writes the FP32 gradient over `logits`."""
    code = _out_code("lmhead_xent_fused", logits if in_place else dlogits, grad_dtype, "fp32")
    pz, ld = _mat(logits, "logits", torch.float32)
    n, V = logits.shape
    pt = _vec(target, "target", torch.int32, n)
    if not isinstance(dloss, torch.Tensor) or not dloss.is_cuda or dloss.dtype != torch.float32:
        raise TypeError("dloss: expected a GPU fp32 tensor")
    _on_current_device(dloss, "dloss")
    if dloss.numel() == 1:
        stride = 0
    elif dloss.numel() == n and dloss.is_contiguous():
        stride = 1
    else:
        raise ValueError("dloss must hold 1 or n_rows contiguous values")
    if stats is None:
        stats = _empty((n, STATS_COLS), torch.float32, logits)
    if loss is None:
        loss = _empty((n,), torch.float32, logits)
    ps = _vec(stats, "stats", torch.float32, n * STATS_COLS)
    pl = _vec(loss, "loss", torch.float32, n) if loss is not False else None
    if in_place:
        dlogits = logits
    elif dlogits is None:
        if code not in (LMH_BF16, LMH_FP32):
            _check("lmhead_xent_fused", 1)
        dlogits = _empty_rows(n, V, _TORCH_DT[code], logits)
    pg, ldg = _mat(dlogits, "dlogits", dlogits.dtype)
    if dlogits.shape != (n, V):
        raise ValueError("dlogits must be [n, V]")
    _check("lmhead_xent_fused",
           lib().lmhead_xent_fused(pz, ld, n, V, pt, int(ignore_index), _vp(dloss.data_ptr()),
                                   stride, pl, ps, pg, ldg, code, _stream(stream)))
    return (loss if loss is not False else None), stats, dlogits


def lmhead_dgrad_workspace_bytes(M, K, V, splits=0):
    """Workspace bytes lmhead_dgrad_ws needs for (M, K, V, splits); 0 = unsplit."""
    n = int(lib().lmhead_dgrad_workspace_bytes(int(M), int(K), int(V), int(splits)))
    if n < 0:
        _check("lmhead_dgrad_workspace_bytes", -n)
    return n


def lmhead_dgrad(dlogits, W, dX=None, dx_dtype=None, splits=0, workspace=None, stream=None):
    """dX[M, K] = dlogits[M, V] . W[V, K] (bf16 operands, fp32 accumulation).

    splits: 0 = the shape's default split of the V sum (lmhead_dgrad_ws; the
    FP32 partials go to `workspace`, a CUDA tensor of at least
    lmhead_dgrad_workspace_bytes(M, K, V, splits) bytes, allocated here from
    torch's caching allocator when not given and marked as in use on the
    launch stream; a raw stream handle needs an explicit workspace),
    1 = the unsplit kernel (lmhead_dgrad), n = n parts.  dx_dtype: the dtype
    of `dX` when given, else 'bf16' unless stated."""
    code = _out_code("lmhead_dgrad", dX, dx_dtype, "bf16")
    pd, ldd = _mat(dlogits, "dlogits", torch.bfloat16)
    pw, ldw = _mat(W, "W", torch.bfloat16)
    M, V = dlogits.shape
    K = W.shape[1]
    if W.shape[0] != V:
        raise ValueError("dlogits and W disagree on V")
    if dX is None:
        if code not in (LMH_BF16, LMH_FP32):
            _check("lmhead_dgrad", 1)
        dX = _empty_rows(M, K, _TORCH_DT[code], dlogits)
    px, ldx = _mat(dX, "dX", dX.dtype)
    if dX.shape != (M, K):
        raise ValueError("dX must be [M, K]")
    splits = int(splits)
    need = 0 if splits == 1 else lmhead_dgrad_workspace_bytes(M, K, V, splits)
    if need == 0:
        _check("lmhead_dgrad", lib().lmhead_dgrad(pd, ldd, pw, ldw, px, ldx, code, M, K, V,
                                                  _stream(stream)))
        return dX
    if workspace is None:
        if stream is not None and not isinstance(stream, torch.cuda.Stream):
            raise ValueError("lmhead_dgrad on a raw stream handle needs an explicit workspace")
        workspace = torch.empty(need, dtype=torch.uint8, device=dlogits.device)
        if stream is not None:
            # freed on return: keep the allocator from reusing it before the
            # kernels on `stream` are done
            workspace.record_stream(stream)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    _on_current_device(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("lmhead_dgrad_ws", lib().lmhead_dgrad_ws(pd, ldd, pw, ldw, px, ldx, code, M, K, V, splits,
                                                    workspace.data_ptr(), nbytes,
                                                    _stream(stream)))
    return dX


def lmhead_dgrad_noalloc(dlogits, W, dX, dx_dtype=None, splits=0, stream=None):
    """lmhead_dgrad with the V-split partial sums in the library's fixed
    per-GPU scratch array (at most DGRAD_NOALLOC_MAX_BYTES) instead of a
    workspace: neither this call nor the library allocates.  dX must be
    passed.  Calls that may overlap on one GPU race on that array."""
    code = _out_code("lmhead_dgrad_noalloc", dX, dx_dtype, "bf16")
    pd, ldd = _mat(dlogits, "dlogits", torch.bfloat16)
    pw, ldw = _mat(W, "W", torch.bfloat16)
    M, V = dlogits.shape
    K = W.shape[1]
    if W.shape[0] != V:
        raise ValueError("dlogits and W disagree on V")
    px, ldx = _mat(dX, "dX", dX.dtype)
    if dX.shape != (M, K):
        raise ValueError("dX must be [M, K]")
    _check("lmhead_dgrad_noalloc",
           lib().lmhead_dgrad_noalloc(pd, ldd, pw, ldw, px, ldx, code, M, K, V, int(splits),
                                      _stream(stream)))
    return dX


def lmhead_wgrad(dlogits, x, dW=None, accumulate=False, stream=None):
    """dW[V, K] (+)= dlogits[M, V]^T . x[M, K] (bf16 operands, fp32 out)."""
    pd, ldd = _mat(dlogits, "dlogits", torch.bfloat16)
    px, ldx = _mat(x, "x", torch.bfloat16)
    M, V = dlogits.shape
    K = x.shape[1]
    if x.shape[0] != M:
        raise ValueError("dlogits and x disagree on M")
    if dW is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing dW")
        dW = _empty_rows(V, K, torch.float32, dlogits)
    pw, ldw = _mat(dW, "dW", torch.float32)
    if dW.shape != (V, K):
        raise ValueError("dW must be [V, K]")
    _check("lmhead_wgrad", lib().lmhead_wgrad(pd, ldd, px, ldx, pw, ldw, int(bool(accumulate)),
                                              M, K, V, _stream(stream)))
    return dW


MFMA_LOOP_FLOP_PER_WORKGROUP_ITER = 2 * 32 * 32 * 16 * 8 * 4  # 8 chains x 4 waves


def lmhead_diag_mfma_loop(iters, n_workgroups, sink=None, stream=None, operands="ones"):
    """Diagnostic register-only MFMA loop; returns sink [n_workgroups * 256]
    FP32.  operands="ones": every element 128 * iters when every MFMA ran;
    operands="random": pseudo-random operands whose sums cancel exactly,
    every element 0 when iters % 4 == 0."""
    iters, n_workgroups = int(iters), int(n_workgroups)
    if operands not in ("ones", "random"):
        raise ValueError("operands must be 'ones' or 'random'")
    if sink is None:
        sink = torch.empty(max(n_workgroups, 0) * 256, dtype=torch.float32, device="cuda")
    if not isinstance(sink, torch.Tensor) or not sink.is_cuda:
        raise TypeError("sink: expected a GPU tensor")
    _on_current_device(sink, "sink")
    if sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < n_workgroups * 256:
        raise ValueError("sink must be a contiguous fp32 tensor of n_workgroups * 256 elements")
    _check("lmhead_diag_mfma_loop",
           lib().lmhead_diag_mfma_loop(iters, n_workgroups, 1 if operands == "random" else 0,
                                       sink.data_ptr(), _stream(stream)))
    return sink
