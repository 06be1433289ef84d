// diag.hip -- a register-only matrix-core loop that measures the sustained
// BF16 MFMA rate of the chip under full matrix load (no memory traffic), so
// that the GEMMs' throughput can be set against what the part actually
// sustains at its power limit, not only against the 2.4 GHz datasheet peak.
//
// Each wave runs CHAINS independent accumulation chains of the 32x32x16 BF16
// MFMA with every operand element 1.0: one MFMA adds 16 to each accumulator
// element, so after `iters` rounds every element holds 16 * iters exactly
// (exact in FP32 while 16 * CHAINS * iters < 2^24).  Each lane writes the sum
// of element 0 of its chains, 16 * CHAINS * iters, which the caller can check.
#include "common.h"

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) mfma_loop_kernel(int64_t iters, float *sink)
{
    // Operands built at run time from `iters` so nothing is a compile-time
    // constant: both are 1.0 for every iters >= 1.
    const float one = iters > 0 ? 1.0f : 0.0f;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(one);
        b[e] = static_cast<__bf16>(one);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[j][e] = 0.0f;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kChains; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
        s += acc[j][0];
    sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

int mfma_loop_chains()
{
    return kChains;
}

hipError_t launch_mfma_loop(int64_t iters, int64_t n_workgroups, float *sink, hipStream_t s)
{
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(static_cast<unsigned>(n_workgroups)), dim3(256), 0,
                       s, iters, sink);
    return hipGetLastError();
}

}  // namespace lmh
