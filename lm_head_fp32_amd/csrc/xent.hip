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

#include <algorithm>

namespace lmh {
#ifndef LMH_XF_PF
#define LMH_XF_PF 1
#endif

namespace {

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

__device__ __forceinline__ float max4(const float4 &v)
{
    return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
}

// The single-read kernel keeps each value's exponential: v <- exp(v - m_t)
// (and the tail value when present), d += every one of them, with m_t the
// thread's own maximum; when m_t = -inf every value is -inf and every e is 0.
// The gradient then needs one multiply per value: exp(z - m) dloss / d =
// e * grad_scale, grad_scale = exp(m_t - m) * dloss / d.
template <int PER>
__device__ __forceinline__ void exp_in_place(float4 (&v)[PER], float &tv, bool has_tail,
                                             float m_t, float &d)
{
    const float ms = (m_t == -INFINITY) ? 0.0f : m_t;  // exp2(-inf) = 0 for every value
    float acc = 0.0f;
    if (has_tail) {
        tv = exp_shifted(tv, ms);
        acc = tv;
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        v[p].x = exp_shifted(v[p].x, ms);
        v[p].y = exp_shifted(v[p].y, ms);
        v[p].z = exp_shifted(v[p].z, ms);
        v[p].w = exp_shifted(v[p].w, ms);
        acc += v[p].x;
        acc += v[p].y;
        acc += v[p].z;
        acc += v[p].w;
    }
    d = acc;
}

__device__ __forceinline__ float grad_scale(float m_t, float m, float d, float up, bool bad)
{
    if (bad)
        return __int_as_float(0x7fc00000);
    const float rescale = (m_t == -INFINITY) ? 0.0f : exp_shifted(m_t, m);
    return rescale * (up / d);
}

// Reduce columns [0, ncols) of one row (16-byte aligned start) to the pair
// (m, d) = (max z, sum exp(z - m)); the result is valid in thread 0.  Each
// thread keeps a running pair over U 16-byte loads at a time (one rescale per
// 4U values), then a wavefront butterfly and a fixed-order cross-wave merge.
template <int NT, int U, bool NTL>
__device__ __forceinline__ void reduce_row_md(const float *zr, int64_t ncols, int tid,
                                              float &m_out, float &d_out)
{
    const float4 *z4 = reinterpret_cast<const float4 *>(zr);
    const int64_t n4 = ncols >> 2;

    float m = -INFINITY, d = 0.0f;
    constexpr int64_t STEP = static_cast<int64_t>(NT) * U;
    auto load_group = [&](float4 (&v)[U], int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * NT + tid;
            v[u] = (i < n4) ? ld4<NTL>(z4 + i)
                            : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
    };
    float4 nxt[U];
    if (LMH_XF_PF && tid < n4)
        load_group(nxt, 0);
    for (int64_t base = 0; base < n4; base += STEP) {
        if (base + tid >= n4)
            break;
        float4 v[U];
        if (LMH_XF_PF) {
            // The next group's loads go out before this group is reduced.
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = nxt[u];
            if (base + STEP + tid < n4)
                load_group(nxt, base + STEP);
        } else {
            load_group(v, base);
        }
        float bm = max4(v[0]);
#pragma unroll
        for (int u = 1; u < U; ++u)
            bm = fmaxf(bm, max4(v[u]));
        const float mn = fmaxf(m, bm);
        // Shift point: mn, or 0 while every value seen is -inf (masked
        // columns): then every term below is exp2(-inf) = 0 and the pair
        // stays empty (m = -inf, d = 0) instead of exp2(-inf + inf) = NaN.
        const float ms = (mn == -INFINITY) ? 0.0f : mn;
        float acc = d * exp_shifted(m, ms);  // m = -inf gives exp2(-inf) = 0
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc += exp_shifted(v[u].x, ms);
            acc += exp_shifted(v[u].y, ms);
            acc += exp_shifted(v[u].z, ms);
            acc += exp_shifted(v[u].w, ms);
        }
        d = acc;
        m = mn;
    }
    // Tail: the last ncols % 4 columns, one per thread.
    {
        const int64_t j = 4 * n4 + tid;
        if (tid < 4 && j < ncols) {
            const float t = zr[j];
            const float mn = fmaxf(m, t);
            const float ms = (mn == -INFINITY) ? 0.0f : mn;
            d = d * exp_shifted(m, ms) + exp_shifted(t, ms);
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
    }
    m_out = m;
    d_out = d;
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
    float m, d;
    reduce_row_md<NT, U, NTL>(zr, V, tid, m, d);
    if (tid == 0) {
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

// Split-vocabulary forward, part 1: one workgroup per (row, column block).
// The slice holds the global columns [col0, col0 + ncols); block b covers its
// columns [b bc, min((b+1) bc, ncols)).  Record {m_b, d_b, X_b, own_b}: own_b
// = 1 and X_b = the target logit when the row's (global) target falls in the
// block, else 0 and 0.
template <int NT, int U, bool NTL>
__global__ __launch_bounds__(NT) void xent_partial_kernel(const float *__restrict__ z, int64_t ld,
                                                          int64_t ncols, int64_t col0, int64_t bc,
                                                          int64_t nb,
                                                          const int32_t *__restrict__ tgt,
                                                          int32_t ignore_index,
                                                          float4 *__restrict__ part,
                                                          int64_t part_stride4)
{
    const int64_t bid = blockIdx.x;
    const int64_t row = bid / nb;
    const int64_t b = bid - row * nb;
    const int tid = threadIdx.x;
    const int64_t j0 = b * bc;
    const int64_t w = min(bc, ncols - j0);
    const float *zb = z + row * ld + j0;
    float m, d;
    reduce_row_md<NT, U, NTL>(zb, w, tid, m, d);
    if (tid == 0) {
        const int32_t y = tgt[row];
        float x = 0.0f, own = 0.0f;
        if (y != ignore_index) {
            const int64_t loc = static_cast<int64_t>(y) - col0 - j0;
            if (loc >= 0 && loc < w) {
                x = zb[loc];
                own = 1.0f;
            }
        }
        part[b * part_stride4 + row] = make_float4(m, d, x, own);
    }
}

// Split-vocabulary forward, part 2: one wavefront per row.  Lane l merges
// the records p = l, l + 64, l + 128, ... in that order into a running pair
// (m, d) (rescaled at each new maximum); the 64 lane pairs are then merged by
// a butterfly, so that m = max m_p and d = sum d_p exp(m_p - m); X_y comes
// from the single owning part.  Writes the same {m, d, X_y, loss} record as
// xent_fwd_kernel.  No owner, several owners or a target outside [0, vocab):
// X_y = loss = NaN.
__global__ __launch_bounds__(256) void xent_merge_kernel(const float4 *__restrict__ part,
                                                         int64_t n_parts, int64_t part_stride4,
                                                         int64_t n_rows,
                                                         const int32_t *__restrict__ tgt,
                                                         int32_t ignore_index, int64_t vocab,
                                                         float *__restrict__ loss,
                                                         float4 *__restrict__ stats)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n_rows)
        return;  // whole wavefronts only: the row is uniform per wave
    float m = -INFINITY, d = 0.0f, x = 0.0f, owners = 0.0f;
    for (int64_t p = lane; p < n_parts; p += 64) {
        const float4 q = part[p * part_stride4 + row];
        merge_md(m, d, q.x, q.y);
        if (q.w != 0.0f) {
            x = q.z;
            owners += q.w;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64), d2 = __shfl_xor(d, off, 64);
        const float x2 = __shfl_xor(x, off, 64), o2 = __shfl_xor(owners, off, 64);
        merge_md(m, d, m2, d2);
        x = (owners != 0.0f) ? x : x2;
        owners += o2;
    }
    if (lane != 0)
        return;
    const int32_t y = tgt[row];
    float l;
    if (y == ignore_index) {
        x = 0.0f;
        l = 0.0f;
    } else if (y < 0 || static_cast<int64_t>(y) >= vocab || owners != 1.0f) {
        x = __int_as_float(0x7fc00000);
        l = x;
    } else {
        l = (m - x) + logf(d);
    }
    stats[row] = make_float4(m, d, x, l);
    if (loss)
        loss[row] = l;
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

// Four -inf values: what the single-read kernel loads for columns past a
// row's end (never written).
__device__ __attribute__((aligned(16))) float kNegInf4[4] = {-INFINITY, -INFINITY, -INFINITY,
                                                            -INFINITY};

// Four FP32 values to four BF16 (two 32-bit words), nearest-even, by the
// hardware's paired conversion.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 bf16x4_rne(const float4 &o)
{
    const f32x2 lo = {o.x, o.y}, hi = {o.z, o.w};
    uint2 w;
    w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
    w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
    return w;
}

// Fused forward + backward for a known upstream gradient: one workgroup per
// row holds the row in registers (PER float4 per thread), so the logits are
// read once.  Each thread reduces its values to a pair (m_t, d_t) and keeps
// e = exp(z - m_t) in place of z; a wave butterfly and, in every wave, a
// butterfly over the waves' pairs give all threads the row's (m, d) with one
// barrier.  Every thread then writes the gradients of exactly the elements it
// read (in place is safe), with the backward kernel's formula: e * scale, and
// fmaf(e, scale, -dloss) at the target column.  Thread 0 writes the forward's
// stats record and loss.
template <int NT, int PER, bool WHOLE, bool OUTBF16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT * 8 / (128 * PER))))
void xent_fused_kernel(const float *z, int64_t ld, int64_t V, const int32_t *__restrict__ tgt,
                       int32_t ignore_index, const float *__restrict__ dloss, int64_t dloss_stride,
                       float *__restrict__ loss, float4 *__restrict__ stats, void *g, int64_t ldg)
{
    static_assert(NT % 64 == 0 && (NT / 64 & (NT / 64 - 1)) == 0 && NT / 64 <= 64, "wave count");
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const float *zr = z + row * ld;
    const float4 *z4 = reinterpret_cast<const float4 *>(zr);
    // WHOLE: V == 4 * NT * PER, every thread holds PER whole float4 and there
    // is no tail.  Otherwise V <= 4 * NT * PER, with a ragged last chunk and
    // up to 3 tail columns.
    const int n4 = WHOLE ? NT * PER : static_cast<int>(V >> 2);
    const int jt = 4 * n4 + tid;  // this thread's tail column (tid < 4)
    const bool has_tail = !WHOLE && tid < 4 && jt < V;
    auto in_row = [&](int p) { return WHOLE || p * NT + tid < n4; };

    // Every load is issued unconditionally, so that the loads stay in flight
    // together: a float4 past the row's end is read from a constant group of
    // four -inf instead (no select on the loaded values, which would make each
    // load wait before the next is issued).
    float4 v[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p)
        v[p] = ld4<true>(in_row(p) ? z4 + p * NT + tid
                                   : reinterpret_cast<const float4 *>(kNegInf4));
    float tv = has_tail ? zr[jt] : -INFINITY;
    const int32_t y = tgt[row];
    const bool ignored = (y == ignore_index);
    const bool bad = !ignored && (y < 0 || static_cast<int64_t>(y) >= V);
    float x = 0.0f;  // the target logit, read by thread 0 before any gradient store
    if (tid == 0 && !ignored && !bad)
        x = zr[y];

    float m = tv;
#pragma unroll
    for (int p = 0; p < PER; ++p)
        m = fmaxf(m, max4(v[p]));
    const float m_t = m;
    float d = 0.0f;
    exp_in_place(v, tv, has_tail, m_t, d);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const float d2 = __shfl_xor(d, off, 64);
        merge_md(m, d, m2, d2);
    }
    // Lane l of every wave takes wave (l mod NW)'s pair; a butterfly over NW
    // lanes leaves every lane with the merge of all NW pairs.  merge_md is
    // symmetric in its two pairs (max, and a sum of two products), so every
    // lane, in every wave, holds the same bits.
    constexpr int NW = NT / 64;
    __shared__ float2 smd[NW];
    __shared__ float sx;
    if ((tid & 63) == 0)
        smd[tid >> 6] = make_float2(m, d);
    if (tid == 0)
        sx = x;  // consumes the load of x before the barrier (in place: no store overtakes it)
    __syncthreads();
    {
        const float2 q = smd[tid & (NW - 1)];
        m = q.x;
        d = q.y;
#pragma unroll
        for (int off = NW / 2; off >= 1; off >>= 1) {
            const float m2 = __shfl_xor(m, off, 64);
            const float d2 = __shfl_xor(d, off, 64);
            merge_md(m, d, m2, d2);
        }
    }
    if (tid == 0) {
        x = sx;
        float l;
        if (ignored) {
            l = 0.0f;
        } else if (bad) {
            x = __int_as_float(0x7fc00000);
            l = x;
        } else {
            l = (m - x) + logf(d);
        }
        stats[row] = make_float4(m, d, x, l);
        if (loss)
            loss[row] = l;
    }

    // Chunk p of the row's gradient starts at a uniform address (p * NT
    // float4); each thread adds only its own index.
    auto store4 = [&](int p, const float4 &o) {
        if constexpr (OUTBF16)
            st2u<true>(reinterpret_cast<uint2 *>(static_cast<uint16_t *>(g) + row * ldg) + p * NT +
                           tid,
                       bf16x4_rne(o));
        else
            st4<true>(reinterpret_cast<float4 *>(static_cast<float *>(g) + row * ldg) + p * NT + tid,
                      o);
    };
    auto store1 = [&](int j, float o) {
        if constexpr (OUTBF16)
            (static_cast<__bf16 *>(g) + row * ldg)[j] = static_cast<__bf16>(o);
        else
            (static_cast<float *>(g) + row * ldg)[j] = o;
    };
    if (ignored) {  // the whole row's gradient is zero, whatever its logits
        const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int p = 0; p < PER; ++p)
            if (in_row(p))
                store4(p, zero);
        if (has_tail)
            store1(jt, 0.0f);
        return;
    }
    const float up = dloss[dloss_stride * row];
    // exp(z - m) / d * dloss = e * exp(m_t - m) * dloss / d (NaN for a bad target)
    const float scale = grad_scale(m_t, m, d, up, bad);
    const int iy = bad ? -1 : (y >> 2);  // the float4 that holds the target column
    const int yl = y & 3;
    if (has_tail)
        store1(jt, (jt == y) ? fmaf(tv, scale, -up) : tv * scale);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        if (!in_row(p))
            break;
        const float4 e = v[p];
        float4 o = make_float4(e.x * scale, e.y * scale, e.z * scale, e.w * scale);
        if (p * NT + tid == iy) {  // one thread of the row
            if (yl == 0)
                o.x = fmaf(e.x, scale, -up);
            else if (yl == 1)
                o.y = fmaf(e.y, scale, -up);
            else if (yl == 2)
                o.z = fmaf(e.z, scale, -up);
            else
                o.w = fmaf(e.w, scale, -up);
        }
        store4(p, o);
    }
}

constexpr int kMeanThreads = 1024;

// Mean of the valid rows' losses and 1/n_valid, in FP64, one workgroup:
// thread t sums rows t, t + 1024, ... in order; each wave combines its 64
// partial sums by a butterfly, and thread 0 adds the 16 wave sums in wave
// order.  A fixed order throughout, so the result is deterministic.
__global__ __launch_bounds__(kMeanThreads) void xent_mean_kernel(const float *__restrict__ loss,
                                                                 const int32_t *__restrict__ tgt,
                                                                 int32_t ignore_index, int64_t n,
                                                                 float *mean_out, float *inv_out)
{
    constexpr int NW = kMeanThreads / 64;
    const int tid = threadIdx.x;
    double s = 0.0;
    int64_t c = 0;
    for (int64_t i = tid; i < n; i += kMeanThreads) {
        if (tgt[i] != ignore_index) {
            if (loss)  // NULL: count only (1 / n_valid)
                s += static_cast<double>(loss[i]);
            ++c;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        s += __shfl_xor(s, off, 64);
        c += __shfl_xor(c, off, 64);
    }
    __shared__ double ws[NW];
    __shared__ int64_t wc[NW];
    if ((tid & 63) == 0) {
        ws[tid >> 6] = s;
        wc[tid >> 6] = c;
    }
    __syncthreads();
    if (tid == 0) {
        double sum = 0.0;
        int64_t nv = 0;
        for (int w = 0; w < NW; ++w) {
            sum += ws[w];
            nv += wc[w];
        }
        if (mean_out)
            *mean_out = nv ? static_cast<float>(sum / static_cast<double>(nv)) : 0.0f;
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

// Work-items per launch are kept at or below 2^31 (the hardware counts a
// grid dimension's work-items in 32 bits): longer calls run as several
// launches over consecutive row ranges, which changes no result since every
// workgroup handles whole rows on its own.
constexpr int64_t kMaxLaunchItems = int64_t{1} << 31;

hipError_t launch_xent_fwd(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                           const int32_t *target, int32_t ignore_index, float *loss, float *stats,
                           hipStream_t s)
{
    if (n_rows == 0)
        return hipSuccess;
    float4 *st = reinterpret_cast<float4 *>(stats);
    const int nt = n_rows < 512 ? 1024 : 256;
    const int64_t chunk = kMaxLaunchItems / nt;
    for (int64_t r0 = 0; r0 < n_rows; r0 += chunk) {
        const unsigned nr = static_cast<unsigned>(std::min(chunk, n_rows - r0));
        const float *z = logits + r0 * ld;
        float *l = loss ? loss + r0 : nullptr;
        if (nt == 1024)
            hipLaunchKernelGGL((xent_fwd_kernel<1024, 4, LMH_XF_NTL>), dim3(nr), dim3(1024), 0, s,
                               z, ld, n_cols, target + r0, ignore_index, l, st + r0);
        else
            hipLaunchKernelGGL((xent_fwd_kernel<256, LMH_XF_U, LMH_XF_NTL>), dim3(nr), dim3(256), 0,
                               s, z, ld, n_cols, target + r0, ignore_index, l, st + r0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_xent_partial(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                               int64_t col0, int64_t block_cols, const int32_t *target,
                               int32_t ignore_index, float *part, int64_t part_stride,
                               hipStream_t s)
{
    if (n_rows == 0)
        return hipSuccess;
    const int64_t nb = (n_cols + block_cols - 1) / block_cols;
    const int64_t max_wg = kMaxLaunchItems / 256;
    // Launch over [rows r0, r0 + nr) x [blocks b0, b0 + nbc): the slice then
    // starts at column b0 * block_cols (global column col0 + b0 * block_cols),
    // so each block keeps its columns and its record slot.
    auto launch = [&](int64_t r0, int64_t nr, int64_t b0, int64_t nbc) {
        const int64_t j0 = b0 * block_cols;
        const int64_t nc = std::min(n_cols - j0, nbc * block_cols);
        hipLaunchKernelGGL((xent_partial_kernel<256, LMH_XF_U, LMH_XF_NTL>),
                           dim3(static_cast<unsigned>(nbc * nr)), dim3(256), 0, s,
                           logits + r0 * ld + j0, ld, nc, col0 + j0, block_cols, nbc, target + r0,
                           ignore_index, reinterpret_cast<float4 *>(part + b0 * part_stride) + r0,
                           part_stride / 4);
        return hipGetLastError();
    };
    if (nb <= max_wg) {
        const int64_t rows_per = max_wg / nb;
        for (int64_t r0 = 0; r0 < n_rows; r0 += rows_per) {
            const hipError_t e = launch(r0, std::min(rows_per, n_rows - r0), 0, nb);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    for (int64_t r = 0; r < n_rows; ++r)
        for (int64_t b0 = 0; b0 < nb; b0 += max_wg) {
            const hipError_t e = launch(r, 1, b0, std::min(max_wg, nb - b0));
            if (e != hipSuccess)
                return e;
        }
    return hipSuccess;
}

hipError_t launch_xent_merge(const float *part, int64_t n_parts, int64_t part_stride,
                             int64_t n_rows, const int32_t *target, int32_t ignore_index,
                             int64_t vocab, float *loss, float *stats, hipStream_t s)
{
    const int64_t chunk = kMaxLaunchItems / 64;  // one wavefront per row
    for (int64_t r0 = 0; r0 < n_rows; r0 += chunk) {
        const int64_t nr = std::min(chunk, n_rows - r0);
        hipLaunchKernelGGL(xent_merge_kernel, dim3(static_cast<unsigned>((nr + 3) / 4)), dim3(256),
                           0, s, reinterpret_cast<const float4 *>(part) + r0, n_parts,
                           part_stride / 4, nr, target + r0, ignore_index, vocab,
                           loss ? loss + r0 : nullptr, reinterpret_cast<float4 *>(stats) + r0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// Rows of at most kFusedMaxCols columns fit in the registers of one
// 1024-thread workgroup (16 float4 per thread); longer rows take the
// two-kernel path (forward, then backward: the logits are read twice).
constexpr int64_t kFusedMaxCols = 65536;

hipError_t launch_xent_fused(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                             const int32_t *target, int32_t ignore_index, const float *dloss,
                             int64_t dloss_stride, float *loss, float *stats, void *dlogits,
                             int64_t ldg, bool bf16_out, hipStream_t s)
{
    if (n_rows == 0)
        return hipSuccess;
    if (n_cols > kFusedMaxCols) {
        const hipError_t e = launch_xent_fwd(logits, ld, n_rows, n_cols, target, ignore_index,
                                             loss, stats, s);
        if (e != hipSuccess)
            return e;
        return launch_xent_bwd(logits, ld, stats, target, ignore_index, dloss, dloss_stride,
                               dlogits, ldg, bf16_out, n_rows, n_cols, s);
    }
    const int64_t chunk = kMaxLaunchItems / 1024;
    const int64_t gsz = bf16_out ? 2 : 4;
    for (int64_t r0 = 0; r0 < n_rows; r0 += chunk) {
        const dim3 grid(static_cast<unsigned>(std::min(chunk, n_rows - r0))), block(1024);
        const float *z = logits + r0 * ld;
        const int32_t *t = target + r0;
        const float *dl = dloss + dloss_stride * r0;
        float *l = loss ? loss + r0 : nullptr;
        float4 *st = reinterpret_cast<float4 *>(stats) + r0;
        void *g = static_cast<char *>(dlogits) + r0 * ldg * gsz;
#define LMH_FUSED_LAUNCH(PER, WHOLE)                                                            \
    do {                                                                                        \
        if (bf16_out)                                                                           \
            hipLaunchKernelGGL((xent_fused_kernel<1024, PER, WHOLE, true>), grid, block, 0, s, z, \
                               ld, n_cols, t, ignore_index, dl, dloss_stride, l, st, g, ldg);   \
        else                                                                                    \
            hipLaunchKernelGGL((xent_fused_kernel<1024, PER, WHOLE, false>), grid, block, 0, s,   \
                               z, ld, n_cols, t, ignore_index, dl, dloss_stride, l, st, g, ldg); \
    } while (0)
        if (n_cols == 4 * 1024 * 8)
            LMH_FUSED_LAUNCH(8, true);
        else if (n_cols < 4 * 1024 * 8)
            LMH_FUSED_LAUNCH(8, false);
        else if (n_cols == 4 * 1024 * 16)
            LMH_FUSED_LAUNCH(16, true);
        else
            LMH_FUSED_LAUNCH(16, false);
#undef LMH_FUSED_LAUNCH
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
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
    const int64_t chunk = std::max<int64_t>(1, kMaxLaunchItems / NT / bpr);
    const int64_t gsz = bf16_out ? 2 : 4;
    const float4 *st = reinterpret_cast<const float4 *>(stats);
    for (int64_t r0 = 0; r0 < n_rows; r0 += chunk) {
        const unsigned nblk = static_cast<unsigned>(bpr * std::min(chunk, n_rows - r0));
        const float *z = logits + r0 * ld;
        const float *dl = dloss + dloss_stride * r0;
        void *g = static_cast<char *>(dlogits) + r0 * ldg * gsz;
        if (bf16_out)
            hipLaunchKernelGGL((xent_bwd_kernel<NT, U, true, LMH_XB_NTL, LMH_XB_NTS>), dim3(nblk),
                               dim3(NT), 0, s, z, ld, st + r0, target + r0, ignore_index, dl,
                               dloss_stride, g, ldg, n_cols, bpr);
        else
            hipLaunchKernelGGL((xent_bwd_kernel<NT, U, false, LMH_XB_NTL, LMH_XB_NTS>), dim3(nblk),
                               dim3(NT), 0, s, z, ld, st + r0, target + r0, ignore_index, dl,
                               dloss_stride, g, ldg, n_cols, bpr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace lmh
