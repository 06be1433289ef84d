// common.h -- internal declarations shared by the gfx950 kernels and the
// C-ABI layer of liblmhead.so.  Not installed; the public interface is
// include/lmhead.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

// Operand description for the generic contraction
//   D[c][r] (op)= sum_p A(r, p) * B(c, p)
// A(r, p) is at A[r * lda + p] when !a_trans (p contiguous) and at
// A[p * lda + r] when a_trans (r contiguous); B likewise with c.
// D is row-major [C x R] with leading dimension ldd (r contiguous).
struct GemmProblem {
    const uint16_t *A;
    int64_t lda;
    const uint16_t *B;
    int64_t ldb;
    void *D;
    int64_t ldd;
    int64_t R, C, P;
    // kStoreF32Stats only (the logits GEMM, R = vocabulary, C = tokens): the
    // tokens' targets and the per-256-row-block cross-entropy records
    // {m, d, X_y, own} written at part4[(r0 / 256) * part_stride4 + c].
    const int32_t *tgt = nullptr;
    int32_t ignore_index = 0;
    void *part4 = nullptr;
    int64_t part_stride4 = 0;
    // Split of the sum over p (gemm_big only): workgroup row blockIdx.y sums
    // p in [y * psplit, min(P, (y + 1) * psplit)) and stores its FP32 partial
    // tile at D + y * split_stride.  psplit == 0: no split.
    int64_t psplit = 0;
    int64_t split_stride = 0;
    // Output stores bypass the caches' normal allocation (nontemporal): a
    // GEMM's output is written once and not read back by this kernel, and
    // lines left dirty in L2 and the 256 MB MALL would otherwise be written
    // back during the next kernel's reads.  Off for partial sums that the
    // next kernel reads back at once.
    bool stream_out = true;
};

typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store16(float *p, float4 v, bool stream)
{
    if (stream) {
        const f32x4_nt w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4_nt *>(p));
    } else {
        *reinterpret_cast<float4 *>(p) = v;
    }
}

typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store8(uint16_t *p, uint2 v, bool stream)
{
    if (stream) {
        const u32x2_nt w = {v.x, v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_nt *>(p));
    } else {
        *reinterpret_cast<uint2 *>(p) = v;
    }
}

__device__ __forceinline__ void store16(uint16_t *p, uint4 v, bool stream)
{
    if (stream) {
        const u32x4_nt w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt *>(p));
    } else {
        *reinterpret_cast<uint4 *>(p) = v;
    }
}

enum class Epi : int { kStoreF32 = 0, kStoreBF16 = 1, kAccumF32 = 2, kStoreF32Stats = 3 };

// Launchers (return the hipError_t of the launch).
hipError_t launch_gemm_logits(const GemmProblem &p, Epi epi, hipStream_t s);
// True when launch_gemm_logits runs kStoreF32Stats in its epilogue for p
// (the 256 x 256 eight-wave kernels); otherwise the caller computes the
// records from the stored logits.
bool gemm_logits_stats_in_epilogue(const GemmProblem &p);
hipError_t launch_gemm_dgrad(const GemmProblem &p, Epi epi, hipStream_t s);
// dgrad with the sum over V split `splits` ways (0 = the shape's default):
// FP32 partials in `ws`, then a reduction in split order into p.D.
int dgrad_default_splits(int64_t M, int64_t K, int64_t V);
int64_t dgrad_workspace_elems(int64_t M, int64_t K, int64_t V, int splits);
hipError_t launch_gemm_dgrad_split(const GemmProblem &p, bool bf16_out, int splits, float *ws,
                                   hipStream_t s);
hipError_t launch_gemm_wgrad(const GemmProblem &p, Epi epi, hipStream_t s);

hipError_t launch_xent_fwd(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                           const int32_t *target, int32_t ignore_index, float *loss,
                           float *stats, hipStream_t s);
hipError_t launch_xent_partial(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                               int64_t col0, int64_t block_cols, const int32_t *target,
                               int32_t ignore_index, float *part, int64_t part_stride,
                               hipStream_t s);
hipError_t launch_xent_merge(const float *part, int64_t n_parts, int64_t part_stride,
                             int64_t n_rows, const int32_t *target, int32_t ignore_index,
                             int64_t vocab, float *loss, float *stats, hipStream_t s);
hipError_t launch_xent_fused(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                             const int32_t *target, int32_t ignore_index, const float *dloss,
                             int64_t dloss_stride, float *loss, float *stats, void *dlogits,
                             int64_t ldg, bool bf16_out, hipStream_t s);
hipError_t launch_xent_mean(const float *loss, const int32_t *target, int32_t ignore_index,
                            int64_t n_rows, float *mean_out, float *inv_out, hipStream_t s);
hipError_t launch_xent_bwd(const float *logits, int64_t ld, const float *stats,
                           const int32_t *target, int32_t ignore_index, const float *dloss,
                           int64_t dloss_stride, void *dlogits, int64_t ldg, bool bf16_out,
                           int64_t n_rows, int64_t n_cols, hipStream_t s);
// Register-only MFMA loop (diagnostic): 256-thread workgroups, one float per
// thread written to sink; all-ones or pseudo-random operands.
int mfma_loop_chains();
hipError_t launch_mfma_loop(int64_t iters, int64_t n_workgroups, bool random_operands,
                            float *sink, hipStream_t s);

// exp(z - m) as one hardware base-2 exponential; the same form everywhere the
// cross-entropy statistics are computed (CE kernels, logits GEMM epilogue).
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_shifted(float z, float m)
{
    return __builtin_amdgcn_exp2f((z - m) * kLog2e);
}

// Merge two partial (m, d) pairs.  A pair with m = -inf is empty.
__device__ __forceinline__ void merge_md(float &m, float &d, float m2, float d2)
{
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY)
        return;  // both empty
    const float s1 = (m == -INFINITY) ? 0.0f : exp_shifted(m, mn);
    const float s2 = (m2 == -INFINITY) ? 0.0f : exp_shifted(m2, mn);
    d = d * s1 + d2 * s2;
    m = mn;
}

// FP32 -> BF16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
// Written as a select (no branch), so that per-element use compiles to
// straight-line code.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet_nan = (u >> 16) | 0x40u;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? quiet_nan : rounded;
}

}  // namespace lmh
