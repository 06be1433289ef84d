// api.hip -- the C ABI of liblmhead.so (declared in include/lmhead.h).
//
// Every entry point validates its arguments on the host before any HIP call
// and returns an LMH_ERR_* code without touching the GPU when they are
// invalid; otherwise it enqueues its kernels on the caller's stream.
#include "lmhead.h"

#include "common.h"

#include <limits.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

// The fixed scratch array of lmhead_dgrad_noalloc: the V-split dgrad's FP32
// partial sums live here instead of in a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side handle, not device memory: kernels and copies
// take the device address that hipGetSymbolAddress returns for the current
// device (scratch_device_address below), never the name itself.
static __device__ __align__(256) float scratch[LMH_DGRAD_NOALLOC_MAX_BYTES / 4];

namespace {

constexpr int64_t kMaxDim = static_cast<int64_t>(INT_MAX);
constexpr int64_t kMaxDiagWorkgroups = 65536;
constexpr int32_t kMaxSplits = 16;

// Vocabulary columns per cross-entropy record of lmhead_logits_xent (the
// logits GEMM's tile height).
constexpr int64_t kLogitsStatsBlock = 256;

// Work-items per kernel launch are kept at or below 2^31: the hardware counts
// a grid dimension's work-items in 32 bits, and the kernels index workgroups
// with 32-bit integers.  The cross-entropy launchers split longer calls into
// row ranges themselves; a GEMM call whose grid would pass the limit is
// refused on the host (LMH_ERR_SHAPE) before anything is enqueued.
constexpr int64_t kMaxLaunchItems = int64_t{1} << 31;

int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

// An upper bound on the work-items of any grid a GEMM with an R x C output
// can launch.  The densest is the few-token logits kernel, 256 work-items per
// 128 x 32 tile; the large-tile kernels use at most 512 per 256 x 128 tile.
// With the contraction split (at most kMaxSplits parts) each part runs
// 256 x 128 tiles and the reduction one work-item per 4 outputs.
bool gemm_grid_fits(int64_t R, int64_t C, bool split)
{
    const int64_t dense = ceil_div(R, 128) * ceil_div(C, 32);  // <= 2^23 * 2^26
    if (dense > kMaxLaunchItems / 256)
        return false;
    if (split) {
        const int64_t parts = ceil_div(R, 256) * ceil_div(C, 128) * kMaxSplits;
        if (parts > kMaxLaunchItems / 512 || C * ceil_div(R, 4) > kMaxLaunchItems)
            return false;
    }
    return true;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool aligned4(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 3u) == 0;
}

// Elements a row-major [rows x cols] matrix with leading dimension ld may
// span: 2^44, far beyond any GPU's memory, so that spans and kernel offsets
// (row * ld, in 64 bits) cannot overflow.
constexpr int64_t kMaxSpanElems = int64_t{1} << 44;

// True when (rows - 1) * ld + cols stays within kMaxSpanElems (rows, cols and
// ld non-negative; computed without overflow).
bool span_fits(int64_t rows, int64_t cols, int64_t ld)
{
    if (rows <= 0 || cols <= 0)
        return true;
    if (ld > kMaxSpanElems || cols > kMaxSpanElems)
        return false;
    return rows == 1 || ld <= (kMaxSpanElems - cols) / (rows - 1);
}

// Byte range [lo, hi) touched by a row-major [rows x cols] matrix (its span
// checked with span_fits first).
struct Span {
    uintptr_t lo, hi;
};

Span span_of(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t esz)
{
    Span s;
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = (rows <= 0 || cols <= 0)
               ? s.lo
               : s.lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * esz);
    return s;
}

bool overlaps(const Span &a, const Span &b)
{
    return a.lo < b.hi && b.lo < a.hi;
}

int32_t launch_status(hipError_t e)
{
    return e == hipSuccess ? LMH_OK : LMH_ERR_LAUNCH;
}

// Common checks of a row-major matrix operand.
int32_t check_matrix(const void *p, int64_t rows, int64_t cols, int64_t ld, int ld_multiple)
{
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim)
        return LMH_ERR_SHAPE;
    if (rows == 0 || cols == 0)
        return LMH_OK;
    if (!p)
        return LMH_ERR_NULL;
    if (ld < cols || !span_fits(rows, cols, ld))
        return LMH_ERR_SHAPE;
    if (!aligned16(p) || (ld % ld_multiple) != 0)
        return LMH_ERR_ALIGN;
    return LMH_OK;
}

#define LMH_TRY(expr)                 \
    do {                              \
        const int32_t _st = (expr);   \
        if (_st != LMH_OK)            \
            return _st;               \
    } while (0)

int32_t check_dtype_out(int32_t dt)
{
    return (dt == LMH_BF16 || dt == LMH_FP32) ? LMH_OK : LMH_ERR_DTYPE;
}

// --------------------------------------------------------------------------
// The per-device address of the fixed scratch array (defined at file scope
// above the namespace), looked up once per device.
constexpr int64_t kScratchBytes = LMH_DGRAD_NOALLOC_MAX_BYTES;
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device, looked up on the first
// call made on that device (with it current) and kept for later calls.
int32_t scratch_device_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return LMH_ERR_LAUNCH;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return LMH_ERR_LAUNCH;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LMH_OK;
}

// Checks shared by the two split-dgrad entry points: operands, outputs and
// their overlaps, and the grid limit (everything but the workspace).
int32_t check_dgrad_split(const void *dlogits, int64_t ldd, const void *W, int64_t ldw,
                          void *dX, int64_t ldx, int32_t dx_dtype, int64_t M, int64_t K,
                          int64_t V)
{
    const int64_t osz = dx_dtype == LMH_FP32 ? 4 : 2;
    LMH_TRY(check_matrix(dX, M, K, ldx, dx_dtype == LMH_FP32 ? 4 : 8));
    LMH_TRY(check_matrix(dlogits, M, V, ldd, 8));
    LMH_TRY(check_matrix(W, V, K, ldw, 8));
    const Span so = span_of(dX, M, K, ldx, osz);
    if (overlaps(so, span_of(dlogits, M, V, ldd, 2)) || overlaps(so, span_of(W, V, K, ldw, 2)))
        return LMH_ERR_ALIAS;
    if (!gemm_grid_fits(K, M, true))
        return LMH_ERR_SHAPE;
    return LMH_OK;
}

int32_t launch_dgrad_split(const void *dlogits, int64_t ldd, const void *W, int64_t ldw,
                           void *dX, int64_t ldx, int32_t dx_dtype, int64_t M, int64_t K,
                           int64_t V, int32_t splits, float *ws, void *stream)
{
    lmh::GemmProblem p;
    p.A = static_cast<const uint16_t *>(W);
    p.lda = ldw;
    p.B = static_cast<const uint16_t *>(dlogits);
    p.ldb = ldd;
    p.D = dX;
    p.ldd = ldx;
    p.R = K;
    p.C = M;
    p.P = V;
    return launch_status(lmh::launch_gemm_dgrad_split(p, dx_dtype != LMH_FP32, splits, ws,
                                                      static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char *lmhead_status_str(int32_t status)
{
    switch (status) {
    case LMH_OK: return "LMH_OK";
    case LMH_ERR_DTYPE: return "LMH_ERR_DTYPE: unsupported element type (bf16 or fp32 only)";
    case LMH_ERR_SHAPE: return "LMH_ERR_SHAPE: bad size, leading dimension or stride";
    case LMH_ERR_NULL: return "LMH_ERR_NULL: required pointer is NULL";
    case LMH_ERR_ALIGN: return "LMH_ERR_ALIGN: pointer or leading dimension misaligned";
    case LMH_ERR_ALIAS: return "LMH_ERR_ALIAS: output overlaps an input";
    case LMH_ERR_LAUNCH: return "LMH_ERR_LAUNCH: kernel launch failed";
    case LMH_ERR_SCRATCH:
        return "LMH_ERR_SCRATCH: needs more scratch than the library's fixed array holds";
    default: return "unknown lmhead status";
    }
}

int32_t lmhead_version(void)
{
    return 104;
}

int32_t lmhead_logits(const void *x, int64_t ldx, const void *W, int64_t ldw, void *out,
                      int64_t ldo, int32_t out_dtype, int64_t M, int64_t K, int64_t V,
                      void *stream)
{
    LMH_TRY(check_dtype_out(out_dtype));
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim)
        return LMH_ERR_SHAPE;
    const int64_t osz = out_dtype == LMH_FP32 ? 4 : 2;
    LMH_TRY(check_matrix(out, M, V, ldo, out_dtype == LMH_FP32 ? 4 : 8));
    if (M == 0 || V == 0)
        return LMH_OK;
    if (K > 0) {
        LMH_TRY(check_matrix(x, M, K, ldx, 8));
        LMH_TRY(check_matrix(W, V, K, ldw, 8));
        const Span so = span_of(out, M, V, ldo, osz);
        if (overlaps(so, span_of(x, M, K, ldx, 2)) || overlaps(so, span_of(W, V, K, ldw, 2)))
            return LMH_ERR_ALIAS;
    }
    if (!gemm_grid_fits(V, M, false))
        return LMH_ERR_SHAPE;
    lmh::GemmProblem p;
    p.A = static_cast<const uint16_t *>(W);
    p.lda = ldw;
    p.B = static_cast<const uint16_t *>(x);
    p.ldb = ldx;
    p.D = out;
    p.ldd = ldo;
    p.R = V;
    p.C = M;
    p.P = K;
    return launch_status(lmh::launch_gemm_logits(
        p, out_dtype == LMH_FP32 ? lmh::Epi::kStoreF32 : lmh::Epi::kStoreBF16,
        static_cast<hipStream_t>(stream)));
}

int32_t lmhead_logits_xent(const void *x, int64_t ldx, const void *W, int64_t ldw, float *out,
                           int64_t ldo, int64_t M, int64_t K, int64_t V, const int32_t *target,
                           int32_t ignore_index, float *part, int64_t part_stride, void *stream)
{
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim)
        return LMH_ERR_SHAPE;
    LMH_TRY(check_matrix(out, M, V, ldo, 4));
    if (M == 0 || V == 0)
        return LMH_OK;
    const int64_t nparts = (V + kLogitsStatsBlock - 1) / kLogitsStatsBlock;
    if (part_stride < 4 * M || !span_fits(nparts, 4 * M, part_stride))
        return LMH_ERR_SHAPE;
    if (!target || !part)
        return LMH_ERR_NULL;
    if (!aligned4(target) || !aligned16(part) || part_stride % 4 != 0)
        return LMH_ERR_ALIGN;
    const Span so = span_of(out, M, V, ldo, 4);
    const Span st = span_of(target, 1, M, M, 4);
    const Span sp = span_of(part, nparts, 4 * M, part_stride, 4);
    if (overlaps(so, st) || overlaps(so, sp) || overlaps(sp, st))
        return LMH_ERR_ALIAS;
    if (K > 0) {
        LMH_TRY(check_matrix(x, M, K, ldx, 8));
        LMH_TRY(check_matrix(W, V, K, ldw, 8));
        const Span sx = span_of(x, M, K, ldx, 2), sw = span_of(W, V, K, ldw, 2);
        if (overlaps(so, sx) || overlaps(so, sw) || overlaps(sp, sx) || overlaps(sp, sw))
            return LMH_ERR_ALIAS;
    }
    if (!gemm_grid_fits(V, M, false))
        return LMH_ERR_SHAPE;
    lmh::GemmProblem p;
    p.A = static_cast<const uint16_t *>(W);
    p.lda = ldw;
    p.B = static_cast<const uint16_t *>(x);
    p.ldb = ldx;
    p.D = out;
    p.ldd = ldo;
    p.R = V;
    p.C = M;
    p.P = K;
    p.tgt = target;
    p.ignore_index = ignore_index;
    p.part4 = part;
    p.part_stride4 = part_stride / 4;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e = lmh::launch_gemm_logits(p, lmh::Epi::kStoreF32Stats, hs);
    if (e != hipSuccess || lmh::gemm_logits_stats_in_epilogue(p))
        return launch_status(e);
    // Kernels without the epilogue: the records from the stored logits.
    return launch_status(lmh::launch_xent_partial(out, ldo, M, V, 0, kLogitsStatsBlock, target,
                                                  ignore_index, part, part_stride, hs));
}

int32_t lmhead_xent_fwd(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                        const int32_t *target, int32_t ignore_index, float *loss, float *stats,
                        void *stream)
{
    if (n_rows < 0 || n_cols < 0 || n_rows > kMaxDim || n_cols > kMaxDim)
        return LMH_ERR_SHAPE;
    if (n_rows == 0)
        return LMH_OK;
    if (n_cols < 1)
        return LMH_ERR_SHAPE;
    LMH_TRY(check_matrix(logits, n_rows, n_cols, ld, 4));
    if (!target || !stats)
        return LMH_ERR_NULL;
    if (!aligned16(stats) || !aligned4(target) || (loss && !aligned4(loss)))
        return LMH_ERR_ALIGN;
    const Span sz = span_of(logits, n_rows, n_cols, ld, 4);
    const Span ss = span_of(stats, n_rows, 4, 4, 4);
    if (overlaps(sz, ss) || overlaps(ss, span_of(target, 1, n_rows, n_rows, 4)))
        return LMH_ERR_ALIAS;
    if (loss) {
        const Span sl = span_of(loss, 1, n_rows, n_rows, 4);
        if (overlaps(sl, sz) || overlaps(sl, ss) || overlaps(sl, span_of(target, 1, n_rows, n_rows, 4)))
            return LMH_ERR_ALIAS;
    }
    return launch_status(lmh::launch_xent_fwd(logits, ld, n_rows, n_cols, target, ignore_index,
                                              loss, stats, static_cast<hipStream_t>(stream)));
}

int32_t lmhead_xent_partial(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                            int64_t col0, int64_t block_cols, const int32_t *target,
                            int32_t ignore_index, float *part, int64_t part_stride,
                            void *stream)
{
    if (n_rows < 0 || n_cols < 0 || n_rows > kMaxDim || n_cols > kMaxDim)
        return LMH_ERR_SHAPE;
    if (n_rows == 0)
        return LMH_OK;
    if (n_cols < 1 || col0 < 0 || col0 > kMaxDim || block_cols < 4 || block_cols > kMaxDim ||
        block_cols % 4 != 0)
        return LMH_ERR_SHAPE;
    LMH_TRY(check_matrix(logits, n_rows, n_cols, ld, 4));
    const int64_t nb = (n_cols + block_cols - 1) / block_cols;
    if (nb > kMaxDim / n_rows || part_stride < 4 * n_rows || !span_fits(nb, 4 * n_rows, part_stride))
        return LMH_ERR_SHAPE;
    if (!target || !part)
        return LMH_ERR_NULL;
    if (!aligned16(part) || part_stride % 4 != 0 || !aligned4(target))
        return LMH_ERR_ALIGN;
    const Span sp = span_of(part, nb, 4 * n_rows, part_stride, 4);
    if (overlaps(sp, span_of(logits, n_rows, n_cols, ld, 4)) ||
        overlaps(sp, span_of(target, 1, n_rows, n_rows, 4)))
        return LMH_ERR_ALIAS;
    return launch_status(lmh::launch_xent_partial(logits, ld, n_rows, n_cols, col0, block_cols,
                                                  target, ignore_index, part, part_stride,
                                                  static_cast<hipStream_t>(stream)));
}

int32_t lmhead_xent_merge(const float *part, int64_t n_parts, int64_t part_stride,
                          int64_t n_rows, const int32_t *target, int32_t ignore_index,
                          int64_t vocab, float *loss, float *stats, void *stream)
{
    if (n_rows < 0 || n_rows > kMaxDim || n_parts < 0 || n_parts > kMaxDim)
        return LMH_ERR_SHAPE;
    if (n_rows == 0)
        return LMH_OK;
    if (n_parts < 1 || vocab < 1 || part_stride < 4 * n_rows ||
        !span_fits(n_parts, 4 * n_rows, part_stride))
        return LMH_ERR_SHAPE;
    if (!part || !target || !stats)
        return LMH_ERR_NULL;
    if (!aligned16(part) || part_stride % 4 != 0 || !aligned16(stats) || !aligned4(target) ||
        (loss && !aligned4(loss)))
        return LMH_ERR_ALIGN;
    const Span sp = span_of(part, n_parts, 4 * n_rows, part_stride, 4);
    const Span st = span_of(target, 1, n_rows, n_rows, 4);
    const Span ss = span_of(stats, n_rows, 4, 4, 4);
    if (overlaps(ss, sp) || overlaps(ss, st))
        return LMH_ERR_ALIAS;
    if (loss) {
        const Span sl = span_of(loss, 1, n_rows, n_rows, 4);
        if (overlaps(sl, sp) || overlaps(sl, st) || overlaps(sl, ss))
            return LMH_ERR_ALIAS;
    }
    return launch_status(lmh::launch_xent_merge(part, n_parts, part_stride, n_rows, target,
                                                ignore_index, vocab, loss, stats,
                                                static_cast<hipStream_t>(stream)));
}

int32_t lmhead_xent_mean(const float *loss, const int32_t *target, int32_t ignore_index,
                         int64_t n_rows, float *mean_out, float *inv_nvalid_out, void *stream)
{
    if (n_rows < 0 || n_rows > kMaxDim)
        return LMH_ERR_SHAPE;
    if (!mean_out && !inv_nvalid_out)
        return LMH_OK;
    if (n_rows > 0 && (!target || (mean_out && !loss)))
        return LMH_ERR_NULL;
    if ((loss && !aligned4(loss)) || (target && !aligned4(target)) ||
        (mean_out && !aligned4(mean_out)) || (inv_nvalid_out && !aligned4(inv_nvalid_out)))
        return LMH_ERR_ALIGN;
    return launch_status(lmh::launch_xent_mean(loss, target, ignore_index, n_rows, mean_out,
                                               inv_nvalid_out, static_cast<hipStream_t>(stream)));
}

int32_t lmhead_xent_fused(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                          const int32_t *target, int32_t ignore_index, const float *dloss,
                          int64_t dloss_stride, float *loss, float *stats, void *dlogits,
                          int64_t ldg, int32_t grad_dtype, void *stream)
{
    LMH_TRY(check_dtype_out(grad_dtype));
    if (n_rows < 0 || n_cols < 0 || n_rows > kMaxDim || n_cols > kMaxDim)
        return LMH_ERR_SHAPE;
    if (dloss_stride != 0 && dloss_stride != 1)
        return LMH_ERR_SHAPE;
    if (n_rows == 0)
        return LMH_OK;
    if (n_cols < 1)
        return LMH_ERR_SHAPE;
    const bool bf16 = grad_dtype == LMH_BF16;
    LMH_TRY(check_matrix(logits, n_rows, n_cols, ld, 4));
    LMH_TRY(check_matrix(dlogits, n_rows, n_cols, ldg, bf16 ? 8 : 4));
    if (!stats || !target || !dloss)
        return LMH_ERR_NULL;
    if (!aligned16(stats) || !aligned4(target) || !aligned4(dloss) || (loss && !aligned4(loss)))
        return LMH_ERR_ALIGN;
    const Span sz = span_of(logits, n_rows, n_cols, ld, 4);
    const Span sg = span_of(dlogits, n_rows, n_cols, ldg, bf16 ? 2 : 4);
    const bool in_place = static_cast<const void *>(dlogits) == static_cast<const void *>(logits);
    if (in_place) {
        if (bf16 || ldg != ld)
            return LMH_ERR_ALIAS;
    } else if (overlaps(sz, sg)) {
        return LMH_ERR_ALIAS;
    }
    const int64_t ndl = dloss_stride == 0 ? 1 : n_rows;
    const Span st = span_of(target, 1, n_rows, n_rows, 4);
    const Span sd = span_of(dloss, 1, ndl, ndl, 4);
    const Span ss = span_of(stats, n_rows, 4, 4, 4);
    if (overlaps(sg, ss) || overlaps(sg, st) || overlaps(sg, sd) || overlaps(ss, sz) ||
        overlaps(ss, st) || overlaps(ss, sd))
        return LMH_ERR_ALIAS;
    if (loss) {
        const Span sl = span_of(loss, 1, n_rows, n_rows, 4);
        if (overlaps(sl, sz) || overlaps(sl, sg) || overlaps(sl, ss) || overlaps(sl, st) ||
            overlaps(sl, sd))
            return LMH_ERR_ALIAS;
    }
    return launch_status(lmh::launch_xent_fused(logits, ld, n_rows, n_cols, target, ignore_index,
                                                dloss, dloss_stride, loss, stats, dlogits, ldg,
                                                bf16, static_cast<hipStream_t>(stream)));
}

int32_t lmhead_xent_bwd(const float *logits, int64_t ld, const float *stats,
                        const int32_t *target, int32_t ignore_index, const float *dloss,
                        int64_t dloss_stride, void *dlogits, int64_t ldg, int32_t grad_dtype,
                        int64_t n_rows, int64_t n_cols, void *stream)
{
    LMH_TRY(check_dtype_out(grad_dtype));
    if (n_rows < 0 || n_cols < 0 || n_rows > kMaxDim || n_cols > kMaxDim)
        return LMH_ERR_SHAPE;
    if (dloss_stride != 0 && dloss_stride != 1)
        return LMH_ERR_SHAPE;
    if (n_rows == 0)
        return LMH_OK;
    if (n_cols < 1)
        return LMH_ERR_SHAPE;
    const bool bf16 = grad_dtype == LMH_BF16;
    LMH_TRY(check_matrix(logits, n_rows, n_cols, ld, 4));
    LMH_TRY(check_matrix(dlogits, n_rows, n_cols, ldg, bf16 ? 8 : 4));
    if (!stats || !target || !dloss)
        return LMH_ERR_NULL;
    if (!aligned16(stats) || !aligned4(target) || !aligned4(dloss))
        return LMH_ERR_ALIGN;
    const Span sz = span_of(logits, n_rows, n_cols, ld, 4);
    const Span sg = span_of(dlogits, n_rows, n_cols, ldg, bf16 ? 2 : 4);
    const bool in_place = static_cast<const void *>(dlogits) == static_cast<const void *>(logits);
    if (in_place) {
        if (bf16 || ldg != ld)
            return LMH_ERR_ALIAS;
    } else if (overlaps(sz, sg)) {
        return LMH_ERR_ALIAS;
    }
    const int64_t ndl = dloss_stride == 0 ? 1 : n_rows;
    if (overlaps(sg, span_of(stats, n_rows, 4, 4, 4)) ||
        overlaps(sg, span_of(target, 1, n_rows, n_rows, 4)) ||
        overlaps(sg, span_of(dloss, 1, ndl, ndl, 4)))
        return LMH_ERR_ALIAS;
    return launch_status(lmh::launch_xent_bwd(logits, ld, stats, target, ignore_index, dloss,
                                              dloss_stride, dlogits, ldg, bf16, n_rows, n_cols,
                                              static_cast<hipStream_t>(stream)));
}

int32_t lmhead_dgrad(const void *dlogits, int64_t ldd, const void *W, int64_t ldw, void *dX,
                     int64_t ldx, int32_t dx_dtype, int64_t M, int64_t K, int64_t V, void *stream)
{
    LMH_TRY(check_dtype_out(dx_dtype));
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim)
        return LMH_ERR_SHAPE;
    const int64_t osz = dx_dtype == LMH_FP32 ? 4 : 2;
    LMH_TRY(check_matrix(dX, M, K, ldx, dx_dtype == LMH_FP32 ? 4 : 8));
    if (M == 0 || K == 0)
        return LMH_OK;
    if (V > 0) {
        LMH_TRY(check_matrix(dlogits, M, V, ldd, 8));
        LMH_TRY(check_matrix(W, V, K, ldw, 8));
        const Span so = span_of(dX, M, K, ldx, osz);
        if (overlaps(so, span_of(dlogits, M, V, ldd, 2)) || overlaps(so, span_of(W, V, K, ldw, 2)))
            return LMH_ERR_ALIAS;
    }
    if (!gemm_grid_fits(K, M, false))
        return LMH_ERR_SHAPE;
    lmh::GemmProblem p;
    p.A = static_cast<const uint16_t *>(W);  // stored [V][K] = [P][R]
    p.lda = ldw;
    p.B = static_cast<const uint16_t *>(dlogits);  // [M][V] = [C][P]
    p.ldb = ldd;
    p.D = dX;
    p.ldd = ldx;
    p.R = K;
    p.C = M;
    p.P = V;
    return launch_status(lmh::launch_gemm_dgrad(
        p, dx_dtype == LMH_FP32 ? lmh::Epi::kStoreF32 : lmh::Epi::kStoreBF16,
        static_cast<hipStream_t>(stream)));
}

int64_t lmhead_dgrad_workspace_bytes(int64_t M, int64_t K, int64_t V, int32_t splits)
{
    // dX [M x K] must fit a matrix's span, which also keeps the size below in range.
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim || splits < 0 ||
        splits > kMaxSplits || !span_fits(M, K + 3, K + 3))
        return -static_cast<int64_t>(LMH_ERR_SHAPE);
    return 4 * lmh::dgrad_workspace_elems(M, K, V, splits);
}

int32_t lmhead_dgrad_ws(const void *dlogits, int64_t ldd, const void *W, int64_t ldw, void *dX,
                        int64_t ldx, int32_t dx_dtype, int64_t M, int64_t K, int64_t V,
                        int32_t splits, void *workspace, int64_t workspace_bytes, void *stream)
{
    LMH_TRY(check_dtype_out(dx_dtype));
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim || splits < 0 ||
        splits > kMaxSplits || workspace_bytes < 0 || !span_fits(M, K + 3, K + 3))
        return LMH_ERR_SHAPE;
    const int64_t need = 4 * lmh::dgrad_workspace_elems(M, K, V, splits);
    if (need == 0)
        return lmhead_dgrad(dlogits, ldd, W, ldw, dX, ldx, dx_dtype, M, K, V, stream);
    LMH_TRY(check_matrix(dX, M, K, ldx, dx_dtype == LMH_FP32 ? 4 : 8));
    LMH_TRY(check_matrix(dlogits, M, V, ldd, 8));
    LMH_TRY(check_matrix(W, V, K, ldw, 8));
    if (!workspace)
        return LMH_ERR_NULL;
    if (!aligned16(workspace))
        return LMH_ERR_ALIGN;
    if (workspace_bytes < need)
        return LMH_ERR_SHAPE;
    Span ws;
    ws.lo = reinterpret_cast<uintptr_t>(workspace);
    ws.hi = ws.lo + static_cast<uintptr_t>(need);
    if (overlaps(ws, span_of(dX, M, K, ldx, dx_dtype == LMH_FP32 ? 4 : 2)) ||
        overlaps(ws, span_of(dlogits, M, V, ldd, 2)) || overlaps(ws, span_of(W, V, K, ldw, 2)))
        return LMH_ERR_ALIAS;
    LMH_TRY(check_dgrad_split(dlogits, ldd, W, ldw, dX, ldx, dx_dtype, M, K, V));
    return launch_dgrad_split(dlogits, ldd, W, ldw, dX, ldx, dx_dtype, M, K, V, splits,
                              static_cast<float *>(workspace), stream);
}

int32_t lmhead_dgrad_noalloc(const void *dlogits, int64_t ldd, const void *W, int64_t ldw,
                             void *dX, int64_t ldx, int32_t dx_dtype, int64_t M, int64_t K,
                             int64_t V, int32_t splits, void *stream)
{
    LMH_TRY(check_dtype_out(dx_dtype));
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim || splits < 0 ||
        splits > kMaxSplits || !span_fits(M, K + 3, K + 3))
        return LMH_ERR_SHAPE;
    const int64_t need = 4 * lmh::dgrad_workspace_elems(M, K, V, splits);
    if (need == 0)
        return lmhead_dgrad(dlogits, ldd, W, ldw, dX, ldx, dx_dtype, M, K, V, stream);
    if (need > kScratchBytes)
        return LMH_ERR_SCRATCH;
    LMH_TRY(check_dgrad_split(dlogits, ldd, W, ldw, dX, ldx, dx_dtype, M, K, V));
    void *ws = nullptr;
    LMH_TRY(scratch_device_address(&ws));
    return launch_dgrad_split(dlogits, ldd, W, ldw, dX, ldx, dx_dtype, M, K, V, splits,
                              static_cast<float *>(ws), stream);
}

int32_t lmhead_wgrad(const void *dlogits, int64_t ldd, const void *x, int64_t ldx, float *dW,
                     int64_t ldw, int32_t accumulate, int64_t M, int64_t K, int64_t V,
                     void *stream)
{
    if (M < 0 || K < 0 || V < 0 || M > kMaxDim || K > kMaxDim || V > kMaxDim)
        return LMH_ERR_SHAPE;
    LMH_TRY(check_matrix(dW, V, K, ldw, 4));
    if (V == 0 || K == 0)
        return LMH_OK;
    if (M == 0 && accumulate)
        return LMH_OK;
    if (M > 0) {
        LMH_TRY(check_matrix(dlogits, M, V, ldd, 8));
        LMH_TRY(check_matrix(x, M, K, ldx, 8));
        const Span so = span_of(dW, V, K, ldw, 4);
        if (overlaps(so, span_of(dlogits, M, V, ldd, 2)) || overlaps(so, span_of(x, M, K, ldx, 2)))
            return LMH_ERR_ALIAS;
    }
    if (!gemm_grid_fits(K, V, false))
        return LMH_ERR_SHAPE;
    lmh::GemmProblem p;
    p.A = static_cast<const uint16_t *>(x);  // stored [M][K] = [P][R]
    p.lda = ldx;
    p.B = static_cast<const uint16_t *>(dlogits);  // stored [M][V] = [P][C]
    p.ldb = ldd;
    p.D = dW;
    p.ldd = ldw;
    p.R = K;
    p.C = V;
    p.P = M;
    return launch_status(lmh::launch_gemm_wgrad(
        p, accumulate ? lmh::Epi::kAccumF32 : lmh::Epi::kStoreF32,
        static_cast<hipStream_t>(stream)));
}

int32_t lmhead_diag_mfma_loop(int64_t iters, int64_t n_workgroups, int32_t operands, float *sink,
                              void *stream)
{
    const int64_t chains = lmh::mfma_loop_chains();
    if (operands != 0 && operands != 1)
        return LMH_ERR_SHAPE;
    if (iters < 0 || n_workgroups < 0 || n_workgroups > kMaxDiagWorkgroups ||
        16 * chains * iters >= (int64_t{1} << 24))
        return LMH_ERR_SHAPE;
    if (n_workgroups == 0)
        return LMH_OK;
    if (!sink)
        return LMH_ERR_NULL;
    if (!aligned16(sink))
        return LMH_ERR_ALIGN;
    return launch_status(lmh::launch_mfma_loop(iters, n_workgroups, operands == 1, sink,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
