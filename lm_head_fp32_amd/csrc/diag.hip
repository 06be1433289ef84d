// diag.hip -- a register-only matrix-core loop that measures the sustained
// BF16 MFMA rate of the chip under full matrix load (no memory traffic), so
// that the GEMMs' throughput can be set against what the part actually
// sustains at its power limit, not only against the 2.4 GHz datasheet peak.
//
// Each wave runs CHAINS independent accumulation chains of the 32x32x16 BF16
// MFMA; one round is one MFMA per chain.  Two operand kinds:
//
//  * all ones: one MFMA adds 16 to each accumulator element, so after `iters`
//    rounds every element holds 16 * iters exactly (exact in FP32 while
//    16 * CHAINS * iters < 2^24).  Almost no operand bit changes from one
//    MFMA to the next, so this measures the pipe at its lowest switching power.
//  * random: every lane holds two operand pairs (A1, B1), (A2, B2) of
//    pseudo-random BF16 values with random sign, exponent 0 and seven random
//    mantissa bits (|v| in [1, 2)), drawn from an integer hash of the thread's
//    global index; the pairs (A1, -B1) and (A2, -B2) complete a cycle of four.
//    Chain j uses pair (r + j) % 4 in round r, so consecutive MFMAs of a wave
//    never share operands and the multipliers switch as on real data.  Every
//    product is a multiple of 2^-14 below 4 in magnitude and every partial sum
//    of a cycle stays below 2^8, so all sums are exact in FP32: each chain is
//    back to exactly 0 after every fourth round.
//
// Each lane writes the sum of element 0 of its chains: 16 * CHAINS * iters for
// all-ones operands.  For random operands the sum is weighted by chain number
// (1 ... CHAINS); it is 0 when iters % 4 == 0, and the same value for every
// iters of one residue mod 4 (the partial cycle).
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

// 32-bit integer hash (the finaliser of MurmurHash3).
__device__ __forceinline__ uint32_t mix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Eight BF16 values with random sign and mantissa, exponent 0, built as four
// 32-bit words of two values each (element 2w in the low half of word w).
__device__ __forceinline__ bf16x8 random_operand(uint32_t seed)
{
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = mix32(seed * 8u + 2u * q);
        const uint32_t hi = mix32(seed * 8u + 2u * q + 1u);
        const uint32_t vlo = ((lo & 0x100u) << 7) | 0x3f80u | (lo & 0x7fu);
        const uint32_t vhi = ((hi & 0x100u) << 7) | 0x3f80u | (hi & 0x7fu);
        w[q] = vlo | (vhi << 16);
    }
    return __builtin_bit_cast(bf16x8, w);
}

// Flips the sign bit of all eight values.
__device__ __forceinline__ bf16x8 negate(bf16x8 v)
{
    u32x4 w = __builtin_bit_cast(u32x4, v);
    w ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, w);
}

__global__ void __launch_bounds__(256) mfma_loop_random_kernel(int64_t iters, float *sink)
{
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    bf16x8 opa[4], opb[4];
    opa[0] = random_operand(4u * gid + 0u);
    opb[0] = random_operand(4u * gid + 1u);
    opa[1] = random_operand(4u * gid + 2u);
    opb[1] = random_operand(4u * gid + 3u);
    opa[2] = opa[0];
    opb[2] = negate(opb[0]);
    opa[3] = opa[1];
    opb[3] = negate(opb[1]);
    f32x16 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[j][e] = 0.0f;
    int64_t i = 0;
    for (; i + 4 <= iters; i += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[(r + j) % 4], opb[(r + j) % 4],
                                                                 acc[j], 0, 0, 0);
    }
    const int rest = static_cast<int>(iters - i);
#pragma unroll
    for (int r = 0; r < 3; ++r)
        if (r < rest)
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[(r + j) % 4], opb[(r + j) % 4],
                                                                 acc[j], 0, 0, 0);
    // Chain sums cancel over a cycle, so the chains are weighted 1 ... 8.
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
        s += static_cast<float>(j + 1) * acc[j][0];
    sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

int mfma_loop_chains()
{
    return kChains;
}

hipError_t launch_mfma_loop(int64_t iters, int64_t n_workgroups, bool random_operands,
                            float *sink, hipStream_t s)
{
    if (random_operands)
        hipLaunchKernelGGL(mfma_loop_random_kernel, dim3(static_cast<unsigned>(n_workgroups)),
                           dim3(256), 0, s, iters, sink);
    else
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(static_cast<unsigned>(n_workgroups)), dim3(256),
                           0, s, iters, sink);
    return hipGetLastError();
}

}  // namespace lmh
