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
};

enum class Epi : int { kStoreF32 = 0, kStoreBF16 = 1, kAccumF32 = 2 };

// Launchers (return the hipError_t of the launch).
hipError_t launch_gemm_logits(const GemmProblem &p, Epi epi, hipStream_t s);
hipError_t launch_gemm_dgrad(const GemmProblem &p, Epi epi, hipStream_t s);
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

// FP32 -> BF16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace lmh
