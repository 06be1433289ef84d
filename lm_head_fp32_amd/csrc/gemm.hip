// gemm.hip -- BF16 x BF16 -> FP32 contraction on gfx950 matrix cores.
//
// One kernel template serves the three GEMMs of the LM head:
//   logits  out[m][v]  = sum_k x[m][k] W[v][k]     (R = V, C = M, P = K)
//   dgrad   dX[m][k]   = sum_v dl[m][v] W[v][k]    (R = K, C = M, P = V)
//   wgrad   dW[v][k] (+)= sum_m dl[m][v] x[m][k]   (R = K, C = V, P = M)
// The logits GEMM keeps the FP32 accumulator as the FP32 output, or rounds
// it to BF16 for the legacy comparison (Megatron-LM "Add mixed-precision
// (FP32) LM output logits", section "What does this PR do?").
//
// Orientation: the kernel computes D^T tiles with the matrix-core "row"
// dimension on R, the output's contiguous dimension.  A 32x32 MFMA leaves
// four consecutive rows of one column in each lane, so every lane stores 16
// contiguous bytes of an output row with no LDS round trip.
//
// Data movement per workgroup and K-stage (BK = 64 contraction elements):
//   global -> registers (16-byte loads, coalesced along the contiguous dim)
//   registers -> LDS, laid out [row][p] with a 16-byte pad per row so the
//   32 rows read by one MFMA operand fetch fall in distinct bank groups;
//   operands stored p-major in HBM (dgrad's W, wgrad's x and dl) are loaded
//   as 8x8 blocks and transposed in registers before the LDS write.
//   LDS is double buffered: the next stage's global loads are in flight
//   while the current stage feeds the MFMAs.
// Workgroup -> tile mapping: consecutive workgroup ids are dealt round-robin
// to the 8 XCDs; ids are regrouped so that the tiles one XCD runs at the same
// time share operand strips in that XCD's L2.
#include "common.h"

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;

struct TileMap {
    int tiles_r, tiles_c, group_r;
};

// Map a hardware workgroup id to (tile_r, tile_c).
__device__ __forceinline__ void map_tile(const TileMap &tm, int &tr, int &tc)
{
    const int nwg = gridDim.x;
    int b = blockIdx.x;
    // Undo the round-robin XCD dealing: ids b, b+8, b+16, ... share an XCD.
    if ((nwg % kXcds) == 0) {
        const int per = nwg / kXcds;
        b = (b % kXcds) * per + b / kXcds;
    }
    // Grouped order: walk group_r tiles down R, then step along C.
    const int gsz = tm.group_r * tm.tiles_c;
    const int g = b / gsz;
    const int first_r = g * tm.group_r;
    const int rows_in_group = min(tm.tiles_r - first_r, tm.group_r);
    const int in = b - g * gsz;
    tr = first_r + in % rows_in_group;
    tc = in / rows_in_group;
}

__device__ __forceinline__ uint4 load16(const uint16_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

// Load up to 8 contiguous BF16 words starting at p, of which n (< 8) are
// valid; the rest are zero.
__device__ __forceinline__ uint4 load_partial(const uint16_t *p, int n)
{
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < n; ++e)
        w[e >> 1] |= static_cast<uint32_t>(p[e]) << ((e & 1) * 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b)
{
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b)
{
    return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t comp(const uint4 &v, int h)
{
    return h == 0 ? v.x : h == 1 ? v.y : h == 2 ? v.z : v.w;
}

// in[e] holds 8 values along the contiguous dim at contraction index e;
// out[j] receives the 8 contraction values of contiguous index j.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8])
{
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        out[2 * h + 0] = make_uint4(lo_pair(comp(in[0], h), comp(in[1], h)),
                                    lo_pair(comp(in[2], h), comp(in[3], h)),
                                    lo_pair(comp(in[4], h), comp(in[5], h)),
                                    lo_pair(comp(in[6], h), comp(in[7], h)));
        out[2 * h + 1] = make_uint4(hi_pair(comp(in[0], h), comp(in[1], h)),
                                    hi_pair(comp(in[2], h), comp(in[3], h)),
                                    hi_pair(comp(in[4], h), comp(in[5], h)),
                                    hi_pair(comp(in[6], h), comp(in[7], h)));
    }
}

// One operand tile: ROWS x BK elements staged in LDS as [row][p] (padded).
template <int ROWS, int BK, int NT, bool TRANS>
struct TileLoader {
    static constexpr int LDK = BK + 8;
    // Direct (p contiguous in HBM): 16-byte chunks, BK/8 per row.
    static constexpr int kChunks = ROWS * BK / 8;
    static constexpr int kPerThread = (kChunks + NT - 1) / NT;
    // Transposed (rows contiguous in HBM): 8x8 blocks.
    static constexpr int kBlocks = (BK / 8) * (ROWS / 8);
    static constexpr int kBlocksPerThread = (kBlocks + NT - 1) / NT;
    static constexpr int kRegs = TRANS ? 8 * kBlocksPerThread : kPerThread;

    uint4 reg[kRegs];

    __device__ __forceinline__ void load(const uint16_t *__restrict__ base, int64_t ld,
                                         int64_t row0, int64_t nrows, int64_t p0, int64_t np,
                                         int tid)
    {
        if constexpr (!TRANS) {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int c = tid + i * NT;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (kChunks % NT == 0 || c < kChunks) {
                    const int r = c / (BK / 8);
                    const int kc = c % (BK / 8);
                    const int64_t gr = row0 + r;
                    const int64_t gp = p0 + kc * 8;
                    if (gr < nrows) {
                        const uint16_t *src = base + gr * ld + gp;
                        if (gp + 8 <= np)
                            v = load16(src);
                        else if (gp < np)
                            v = load_partial(src, static_cast<int>(np - gp));
                    }
                }
                reg[i] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kBlocksPerThread; ++i) {
                const int blk = tid + i * NT;
                const bool live = (kBlocks % NT == 0) || blk < kBlocks;
                const int pg = blk / (ROWS / 8);
                const int rg = blk % (ROWS / 8);
                const int64_t gr = row0 + rg * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint4 v = make_uint4(0u, 0u, 0u, 0u);
                    const int64_t gp = p0 + pg * 8 + e;
                    if (live && gp < np && gr < nrows) {
                        const uint16_t *src = base + gp * ld + gr;
                        if (gr + 8 <= nrows)
                            v = load16(src);
                        else
                            v = load_partial(src, static_cast<int>(nrows - gr));
                    }
                    reg[i * 8 + e] = v;
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t *lds, int tid)
    {
        if constexpr (!TRANS) {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int c = tid + i * NT;
                if (kChunks % NT == 0 || c < kChunks) {
                    const int r = c / (BK / 8);
                    const int kc = c % (BK / 8);
                    *reinterpret_cast<uint4 *>(lds + r * LDK + kc * 8) = reg[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kBlocksPerThread; ++i) {
                const int blk = tid + i * NT;
                if ((kBlocks % NT == 0) || blk < kBlocks) {
                    const int pg = blk / (ROWS / 8);
                    const int rg = blk % (ROWS / 8);
                    uint4 in[8], out[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        in[e] = reg[i * 8 + e];
                    transpose8x8(in, out);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        *reinterpret_cast<uint4 *>(lds + (rg * 8 + j) * LDK + pg * 8) = out[j];
                }
            }
        }
    }
};

template <int BR, int BC, int BK, int WR, int WC, bool AT, bool BT, int EPI>
__global__ __launch_bounds__(WR * WC * 64) void gemm_kernel(GemmProblem g, TileMap tm)
{
    constexpr int NT = WR * WC * 64;
    constexpr int TR = BR / WR;  // wave tile along R
    constexpr int TC = BC / WC;  // wave tile along C
    constexpr int FR = TR / 32;
    constexpr int FC = TC / 32;
    constexpr int LDK = BK + 8;
    static_assert(TR % 32 == 0 && TC % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BK % 16 == 0, "BK must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BR * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BC * LDK];

    int tr, tc;
    map_tile(tm, tr, tc);
    const int64_t r0 = static_cast<int64_t>(tr) * BR;
    const int64_t c0 = static_cast<int64_t>(tc) * BC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave % WR;
    const int wc = wave / WR;

    TileLoader<BR, BK, NT, AT> la;
    TileLoader<BC, BK, NT, BT> lb;

    f32x16 acc[FR][FC];
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FC; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    const int64_t nk = (g.P + BK - 1) / BK;
    if (nk > 0) {
        la.load(g.A, g.lda, r0, g.R, 0, g.P, tid);
        lb.load(g.B, g.ldb, c0, g.C, 0, g.P, tid);
        la.store(sA[0], tid);
        lb.store(sB[0], tid);
        __syncthreads();
    }

    const int lrow = lane & 31;
    const int lk = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(g.A, g.lda, r0, g.R, (kt + 1) * BK, g.P, tid);
            lb.load(g.B, g.ldb, c0, g.C, (kt + 1) * BK, g.P, tid);
        }
        const uint16_t *a_s = sA[cur] + (wr * TR + lrow) * LDK + lk;
        const uint16_t *b_s = sB[cur] + (wc * TC + lrow) * LDK + lk;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 af[FR], bfr[FC];
#pragma unroll
            for (int i = 0; i < FR; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(a_s + i * 32 * LDK + kk);
#pragma unroll
            for (int j = 0; j < FC; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(b_s + j * 32 * LDK + kk);
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int j = 0; j < FC; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (more) {
            la.store(sA[cur ^ 1], tid);
            lb.store(sB[cur ^ 1], tid);
        }
        __syncthreads();
    }

    // Epilogue.  Lane l, accumulator register 4q+e of a 32x32 tile holds
    // row 8q + 4(l/32) + e, column l%32.
#pragma unroll
    for (int i = 0; i < FR; ++i) {
#pragma unroll
        for (int j = 0; j < FC; ++j) {
            const int64_t c = c0 + wc * TC + j * 32 + (lane & 31);
            if (c >= g.C)
                continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = r0 + wr * TR + i * 32 + q * 8 + (lane >> 5) * 4;
                if (r >= g.R)
                    continue;
                const float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                const bool full = r + 4 <= g.R;
                if constexpr (EPI == static_cast<int>(Epi::kStoreBF16)) {
                    uint16_t *out = static_cast<uint16_t *>(g.D) + c * g.ldd + r;
                    if (full) {
                        uint2 w;
                        w.x = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
                        w.y = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
                        *reinterpret_cast<uint2 *>(out) = w;
                    } else {
                        const float vv[4] = {v0, v1, v2, v3};
                        for (int e = 0; e < 4 && r + e < g.R; ++e)
                            out[e] = static_cast<uint16_t>(f32_to_bf16_bits(vv[e]));
                    }
                } else {
                    float *out = static_cast<float *>(g.D) + c * g.ldd + r;
                    if (full) {
                        float4 w = make_float4(v0, v1, v2, v3);
                        if constexpr (EPI == static_cast<int>(Epi::kAccumF32)) {
                            const float4 o = *reinterpret_cast<const float4 *>(out);
                            w.x += o.x, w.y += o.y, w.z += o.z, w.w += o.w;
                        }
                        *reinterpret_cast<float4 *>(out) = w;
                    } else {
                        const float vv[4] = {v0, v1, v2, v3};
                        for (int e = 0; e < 4 && r + e < g.R; ++e) {
                            if constexpr (EPI == static_cast<int>(Epi::kAccumF32))
                                out[e] = out[e] + vv[e];
                            else
                                out[e] = vv[e];
                        }
                    }
                }
            }
        }
    }
}

template <int BR, int BC, int WR, int WC, bool AT, bool BT>
hipError_t launch_cfg(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    constexpr int BK = 64;
    TileMap tm;
    tm.tiles_r = static_cast<int>((p.R + BR - 1) / BR);
    tm.tiles_c = static_cast<int>((p.C + BC - 1) / BC);
    tm.group_r = group_r < 1 ? 1 : group_r;
    const int64_t nwg = static_cast<int64_t>(tm.tiles_r) * tm.tiles_c;
    if (nwg == 0)
        return hipSuccess;
    dim3 grid(static_cast<unsigned>(nwg)), block(WR * WC * 64);
    switch (epi) {
    case Epi::kStoreF32:
        hipLaunchKernelGGL((gemm_kernel<BR, BC, BK, WR, WC, AT, BT, 0>), grid, block, 0, s, p, tm);
        break;
    case Epi::kStoreBF16:
        hipLaunchKernelGGL((gemm_kernel<BR, BC, BK, WR, WC, AT, BT, 1>), grid, block, 0, s, p, tm);
        break;
    case Epi::kAccumF32:
        hipLaunchKernelGGL((gemm_kernel<BR, BC, BK, WR, WC, AT, BT, 2>), grid, block, 0, s, p, tm);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_logits(const GemmProblem &p, Epi epi, hipStream_t s)
{
    // R = V (vocabulary), C = M (tokens).
    if (p.C <= 32)
        return launch_cfg<128, 32, 4, 1, false, false>(p, epi, 8, s);
    return launch_cfg<128, 128, 2, 2, false, false>(p, epi, 8, s);
}

hipError_t launch_gemm_dgrad(const GemmProblem &p, Epi epi, hipStream_t s)
{
    // R = K (hidden), C = M (tokens), A = W stored [V][K] (transposed).
    return launch_cfg<128, 128, 2, 2, true, false>(p, epi, 8, s);
}

hipError_t launch_gemm_wgrad(const GemmProblem &p, Epi epi, hipStream_t s)
{
    // R = K (hidden), C = V (vocabulary); both operands stored [M][*].
    return launch_cfg<128, 128, 2, 2, true, true>(p, epi, 8, s);
}

}  // namespace lmh
