// xent.hip -- fused vocabulary cross-entropy over FP32 logits on gfx950.
//
// Follows Transformer Engine issue "[Pytorch] change fused cross entropy
// backward grad to fp32 and reduce one read/...": the forward reads the
// logits once and keeps a per-row n_rows x 4 record m_d_X_y (here
// {m, d, X_y, loss}) for the backward (discussion); the backward computes
// the gradient in FP32 (sections "Description", "Changes") and can write it
// over the logits (the original kernel's memory-saving goal, discussion).
//
// Forward, per row i:  m = max_j z_j,  d = sum_j exp(z_j - m)  in ONE pass
//   (online: each thread keeps (m, d) and rescales d by exp(m_old - m_new)
//   once per batch of 4*U values), X = z_y, loss = (m - X) + log d.
// Backward:  g_j = dloss_i * exp(z_j - m) / d  - [j == y] * dloss_i.
//
// Both kernels are HBM-bound streams: 16-byte loads per lane, U loads in
// flight per thread before any arithmetic, no LDS except the final
// cross-wave merge.  exp uses the hardware base-2 exponential on
// (z - m) * log2(e); the subtraction comes first so arguments near zero
// (the large probabilities) carry no cancellation error.
#include "common.h"

#include <math.h>

namespace lmh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte load / store of four FP32 values, optionally marked non-temporal
// (streamed once: do not keep the lines in the caches).
template <bool NT>
__device__ __forceinline__ float4 ld4(const float4 *p)
{
    if constexpr (NT) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}
template <bool NT>
__device__ __forceinline__ void st4(float4 *p, const float4 &v)
{
    if constexpr (NT) {
        const f32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(p));
    } else {
        *p = v;
    }
}
template <bool NT>
__device__ __forceinline__ void st2u(uint2 *p, const uint2 &v)
{
    if constexpr (NT) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = {v.x, v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
    } else {
        *p = v;
    }
}

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

__device__ __forceinline__ float max4(const float4 &v)
{
    return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
}

template <int NT, int U, bool NTL>
__global__ __launch_bounds__(NT) void xent_fwd_kernel(const float *__restrict__ z, int64_t ld,
                                                      int64_t V, const int32_t *__restrict__ tgt,
                                                      int32_t ignore_index, float *__restrict__ loss,
                                                      float4 *__restrict__ stats)
{
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const float *zr = z + row * ld;
    const float4 *z4 = reinterpret_cast<const float4 *>(zr);
    const int64_t n4 = V >> 2;

    float m = -INFINITY, d = 0.0f;
    for (int64_t base = 0; base < n4; base += static_cast<int64_t>(NT) * U) {
        if (base + tid >= n4)
            break;
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * NT + tid;
            v[u] = (i < n4) ? ld4<NTL>(z4 + i)
                            : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
        float bm = max4(v[0]);
#pragma unroll
        for (int u = 1; u < U; ++u)
            bm = fmaxf(bm, max4(v[u]));
        const float mn = fmaxf(m, bm);
        float acc = d * exp_shifted(m, mn);  // m = -inf gives exp2(-inf) = 0
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc += exp_shifted(v[u].x, mn);
            acc += exp_shifted(v[u].y, mn);
            acc += exp_shifted(v[u].z, mn);
            acc += exp_shifted(v[u].w, mn);
        }
        d = acc;
        m = mn;
    }
    // Tail: the last V % 4 columns, one per thread.
    {
        const int64_t j = 4 * n4 + tid;
        if (tid < 4 && j < V) {
            const float t = zr[j];
            const float mn = fmaxf(m, t);
            d = d * exp_shifted(m, mn) + exp_shifted(t, mn);
            m = mn;
        }
    }

    // Wavefront butterfly: every lane ends with the same (m, d).
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const float d2 = __shfl_xor(d, off, 64);
        merge_md(m, d, m2, d2);
    }
    constexpr int NW = NT / 64;
    __shared__ float sm[NW], sd[NW];
    if ((tid & 63) == 0) {
        sm[tid >> 6] = m;
        sd[tid >> 6] = d;
    }
    __syncthreads();
    if (tid == 0) {
        m = sm[0];
        d = sd[0];
        for (int w = 1; w < NW; ++w)
            merge_md(m, d, sm[w], sd[w]);
        const int32_t y = tgt[row];
        float x, l;
        if (y == ignore_index) {
            x = 0.0f;
            l = 0.0f;
        } else if (y < 0 || static_cast<int64_t>(y) >= V) {
            x = __int_as_float(0x7fc00000);
            l = x;
        } else {
            x = zr[y];
            l = (m - x) + logf(d);
        }
        stats[row] = make_float4(m, d, x, l);
        if (loss)
            loss[row] = l;
    }
}

// Gradient of one row chunk.  OUTBF16 selects the store type only; the FP32
// value is computed identically in both instantiations.
template <int NT, int U, bool OUTBF16, bool NTL, bool NTS>
__global__ __launch_bounds__(NT) void xent_bwd_kernel(const float *z, int64_t ld,
                                                      const float4 *__restrict__ stats,
                                                      const int32_t *__restrict__ tgt,
                                                      int32_t ignore_index,
                                                      const float *__restrict__ dloss,
                                                      int64_t dloss_stride, void *g, int64_t ldg,
                                                      int64_t V, int64_t blocks_per_row)
{
    const int64_t bid = blockIdx.x;
    const int64_t row = bid / blocks_per_row;
    const int64_t chunk = bid - row * blocks_per_row;
    const int tid = threadIdx.x;
    const int64_t n4 = V >> 2;

    const int32_t y = tgt[row];
    const bool ignored = (y == ignore_index);
    const bool bad = !ignored && (y < 0 || static_cast<int64_t>(y) >= V);
    const float4 st = stats[row];
    const float m = st.x;
    const float up = ignored ? 0.0f : dloss[dloss_stride * row];
    const float coef = bad ? __int_as_float(0x7fc00000) : up / st.y;

    const float *zr = z + row * ld;
    const float4 *z4 = reinterpret_cast<const float4 *>(zr);

    const int64_t first = chunk * static_cast<int64_t>(NT) * U;
    float4 v[U];
    if (!ignored) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = first + u * NT + tid;
            if (i < n4)
                v[u] = ld4<NTL>(z4 + i);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = first + u * NT + tid;
        if (i >= n4)
            continue;
        float4 o;
        if (ignored) {
            o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        } else {
            // Each lane picks its own value with a select; the target column
            // gets the one-hot term folded in by a single fused multiply-add.
            // Written without branches on purpose: a branching form that wrote
            // one of four lanes was compiled into code that placed the target
            // term in the wrong lane at one unroll factor.
            const int64_t e = static_cast<int64_t>(y) - 4 * i;
            const float ex = exp_shifted(v[u].x, m), ey = exp_shifted(v[u].y, m);
            const float ez = exp_shifted(v[u].z, m), ew = exp_shifted(v[u].w, m);
            o.x = (e == 0) ? fmaf(ex, coef, -up) : ex * coef;
            o.y = (e == 1) ? fmaf(ey, coef, -up) : ey * coef;
            o.z = (e == 2) ? fmaf(ez, coef, -up) : ez * coef;
            o.w = (e == 3) ? fmaf(ew, coef, -up) : ew * coef;
        }
        if constexpr (OUTBF16) {
            uint2 w;
            w.x = f32_to_bf16_bits(o.x) | (f32_to_bf16_bits(o.y) << 16);
            w.y = f32_to_bf16_bits(o.z) | (f32_to_bf16_bits(o.w) << 16);
            st2u<NTS>(reinterpret_cast<uint2 *>(static_cast<uint16_t *>(g) + row * ldg) + i, w);
        } else {
            st4<NTS>(reinterpret_cast<float4 *>(static_cast<float *>(g) + row * ldg) + i, o);
        }
    }
    // Tail: last V % 4 columns, handled by the row's last chunk.
    if (chunk == blocks_per_row - 1 && tid < 4) {
        const int64_t j = 4 * n4 + tid;
        if (j < V) {
            float o = 0.0f;
            if (!ignored) {
                const float e = exp_shifted(zr[j], m);
                o = (j == static_cast<int64_t>(y)) ? fmaf(e, coef, -up) : e * coef;
            }
            if constexpr (OUTBF16)
                (static_cast<uint16_t *>(g) + row * ldg)[j] =
                    static_cast<uint16_t>(f32_to_bf16_bits(o));
            else
                (static_cast<float *>(g) + row * ldg)[j] = o;
        }
    }
}

constexpr int kMeanThreads = 1024;

__global__ __launch_bounds__(kMeanThreads) void xent_mean_kernel(const float *__restrict__ loss,
                                                                 const int32_t *__restrict__ tgt,
                                                                 int32_t ignore_index, int64_t n,
                                                                 float *mean_out, float *inv_out)
{
    const int tid = threadIdx.x;
    double s = 0.0;
    long long c = 0;
    for (int64_t i = tid; i < n; i += kMeanThreads) {
        if (tgt[i] != ignore_index) {
            s += static_cast<double>(loss[i]);
            ++c;
        }
    }
    __shared__ double ss[kMeanThreads];
    __shared__ long long sc[kMeanThreads];
    ss[tid] = s;
    sc[tid] = c;
    __syncthreads();
    for (int w = kMeanThreads / 2; w > 0; w >>= 1) {
        if (tid < w) {
            ss[tid] += ss[tid + w];
            sc[tid] += sc[tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        const long long nv = sc[0];
        if (mean_out)
            *mean_out = nv ? static_cast<float>(ss[0] / static_cast<double>(nv)) : 0.0f;
        if (inv_out)
            *inv_out = nv ? static_cast<float>(1.0 / static_cast<double>(nv)) : 0.0f;
    }
}

}  // namespace

// Launch shapes, chosen by timing on 8192 x 131072 FP32 logits (overridable at
// build time for sweeps).  Both kernels stream every byte once, so the loads of
// the forward pass and the loads and stores of the backward pass are marked
// non-temporal.  Forward: one 256-thread block per row, four 16-byte loads in
// flight per thread.  Backward: 128-thread blocks, each owning 2 x 128 float4
// of one row, which keeps enough small blocks resident to cover HBM latency.
#ifndef LMH_XF_U
#define LMH_XF_U 4
#endif
#ifndef LMH_XF_NTL
#define LMH_XF_NTL true
#endif
#ifndef LMH_XB_NT
#define LMH_XB_NT 128
#endif
#ifndef LMH_XB_U
#define LMH_XB_U 2
#endif
#ifndef LMH_XB_NTL
#define LMH_XB_NTL true
#endif
#ifndef LMH_XB_NTS
#define LMH_XB_NTS true
#endif

hipError_t launch_xent_fwd(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                           const int32_t *target, int32_t ignore_index, float *loss, float *stats,
                           hipStream_t s)
{
    if (n_rows == 0)
        return hipSuccess;
    float4 *st = reinterpret_cast<float4 *>(stats);
    if (n_rows < 512) {
        hipLaunchKernelGGL((xent_fwd_kernel<1024, 4, LMH_XF_NTL>),
                           dim3(static_cast<unsigned>(n_rows)), dim3(1024), 0, s, logits, ld, n_cols,
                           target, ignore_index, loss, st);
    } else {
        hipLaunchKernelGGL((xent_fwd_kernel<256, LMH_XF_U, LMH_XF_NTL>),
                           dim3(static_cast<unsigned>(n_rows)), dim3(256), 0, s, logits, ld, n_cols,
                           target, ignore_index, loss, st);
    }
    return hipGetLastError();
}

hipError_t launch_xent_mean(const float *loss, const int32_t *target, int32_t ignore_index,
                            int64_t n_rows, float *mean_out, float *inv_out, hipStream_t s)
{
    hipLaunchKernelGGL(xent_mean_kernel, dim3(1), dim3(kMeanThreads), 0, s, loss, target,
                       ignore_index, n_rows, mean_out, inv_out);
    return hipGetLastError();
}

hipError_t launch_xent_bwd(const float *logits, int64_t ld, const float *stats,
                           const int32_t *target, int32_t ignore_index, const float *dloss,
                           int64_t dloss_stride, void *dlogits, int64_t ldg, bool bf16_out,
                           int64_t n_rows, int64_t n_cols, hipStream_t s)
{
    if (n_rows == 0)
        return hipSuccess;
    constexpr int NT = LMH_XB_NT, U = LMH_XB_U;
    const int64_t n4 = n_cols >> 2;
    int64_t bpr = (n4 + NT * U - 1) / (NT * U);
    if (bpr < 1)
        bpr = 1;  // rows shorter than 4 columns still need the tail block
    const int64_t nblk = bpr * n_rows;
    const float4 *st = reinterpret_cast<const float4 *>(stats);
    if (bf16_out)
        hipLaunchKernelGGL((xent_bwd_kernel<NT, U, true, LMH_XB_NTL, LMH_XB_NTS>),
                           dim3(static_cast<unsigned>(nblk)), dim3(NT), 0, s, logits, ld, st, target,
                           ignore_index, dloss, dloss_stride, dlogits, ldg, n_cols, bpr);
    else
        hipLaunchKernelGGL((xent_bwd_kernel<NT, U, false, LMH_XB_NTL, LMH_XB_NTS>),
                           dim3(static_cast<unsigned>(nblk)), dim3(NT), 0, s, logits, ld, st, target,
                           ignore_index, dloss, dloss_stride, dlogits, ldg, n_cols, bpr);
    return hipGetLastError();
}

}  // namespace lmh
