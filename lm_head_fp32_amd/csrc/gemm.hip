// gemm.hip -- BF16 x BF16 -> FP32 contractions on gfx950 matrix cores.
//
// The three GEMMs of the LM head, all as D[c][r] = sum_p A(r, p) B(c, p)
// with r the output's contiguous dimension:
//   logits  out[m][v]   = sum_k x[m][k] W[v][k]    (R = V, C = M, P = K)
//   dgrad   dX[m][k]    = sum_v dl[m][v] W[v][k]   (R = K, C = M, P = V)
//   wgrad   dW[v][k] (+)= sum_m dl[m][v] x[m][k]   (R = K, C = V, P = M)
// The logits GEMM keeps the FP32 accumulator as the FP32 output, or rounds
// it to BF16 for the legacy comparison (Megatron-LM "Add mixed-precision
// (FP32) LM output logits", section "What does this PR do?").
//
// Orientation: tiles are computed with the matrix-core "row" dimension on R,
// so a 32x32 MFMA leaves four consecutive output elements of one row in each
// lane; the epilogues stage 32 output rows at a time through LDS and store
// whole rows.
//
// Kernels:
//  * gemm_pp -- the logits GEMM with many tokens and K <= 2048 (or at most
//    384 tokens): 256 x 256 tiles, two wave groups one phase apart over a
//    four-stage LDS ring.
//  * gemm_persist -- wgrad and the many-token logits GEMM over whole tiles:
//    persistent, the next tile's loads and MFMAs overlapping the finished
//    tile's stores.
//  * gemm_wg2 -- wgrad for few tokens otherwise: 256 x 128 tiles, two
//    workgroups per CU.
//  * gemm_big -- 256 x 256 / 256 x 128 / 128 x 128 tiles, two LDS stages fed
//    by direct buffer loads; the logits GEMM for K >= 4096, and dgrad and wgrad
//    (p-major operands read through transposing LDS loads).
//  * gemm_small -- the logits GEMM for few tokens (W streamed once).
//  * gemm_rows -- the logits GEMM for at most 16 tokens and K >= 8192: W
//    streamed 32 rows at a time, K split across the waves.
//  * splitk_reduce -- adds dgrad's FP32 partial sums (V split) in order.
//  * gemm_kernel -- the generic register-staged form, used only when an
//    operand's byte offsets exceed the 32-bit range of buffer loads.
// Workgroup -> tile mapping: the hardware deals consecutive workgroup ids
// round-robin to the 8 XCDs; ids are regrouped so that the tiles one XCD runs
// at the same time share operand strips in that XCD's L2.
#include "common.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------------------
// LDS stage layout of a contraction-contiguous operand (W [V][K], x [M][K],
// dlogits [M][V] in dgrad): [row][BK] BF16, the 16-byte chunk c of row r kept
// at chunk c ^ lds_swz(r).  An MFMA fragment read (ds_read_b128) has lane l
// read row r0 + l % 32 at chunk (2 kk + l / 32) ^ lds_swz(row), and a direct
// load writes 1 KiB linearly, so only the reads depend on the key.  Keys that
// XOR the row's low bits with its higher bits ((r ^ r >> 3) & 7 for 128-byte
// rows) leave those reads free of bank conflicts; the rotation
// (r + (r >> 3)) & 7 used before cost ~4 stall cycles per read in the
// persistent logits kernel (rocprofv3 SQ_LDS_BANK_CONFLICT: 50.3 M cycles
// per launch at M=1024 K=8192 V=32768 -> 0, LDS busy cycles halved, the
// launch 3 % shorter).  Over any 32-row aligned block the key is that of rows
// 0 - 31 XOR a constant of the block, so every fragment reads as the first
// does; for 128-byte rows the constant is 4 x (block parity).
template <int BK>
__device__ __forceinline__ int lds_swz(int row)
{
    static_assert(BK == 64 || BK == 128, "swizzle defined for 128- and 256-byte rows");
    if constexpr (BK == 64)
        return (row ^ (row >> 3)) & 7;
    else
        return (row ^ (row >> 4)) & 15;
}

__device__ __forceinline__ void lds_barrier()
{
    // LDS writes of this wave are complete, then the workgroup barrier; the
    // "memory" clobber keeps the compiler from moving LDS accesses across it.
    // Outstanding global loads (the next stage's prefetch) are not waited on.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x8;
constexpr int kSgVmemRead = 0x20;
constexpr int kSgDsRead = 0x100;

// Buffer resource over one operand tile: base = the tile's first row, range
// checking off in practice (2^31 - 1 bytes); word 3 is the raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base)
{
    // The base is the same for the whole workgroup; say so, so that the
    // descriptor lives in scalar registers.
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void *u = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, static_cast<short>(0), 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff)
{
    auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), soff, 0);
    return *reinterpret_cast<uint4 *>(&v);
}

#define LMH_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// ---------------------------------------------------------------------------
// Operand loaders of gemm_big.  Both fill the same LDS layout: [row][BK] BF16,
// 16-byte chunks XOR-swizzled by row (lds_swz), so the MFMA fragment reads
// are identical whichever way an operand is stored in memory.

// An operand stored [rows][P] (contraction contiguous): each wave instruction
// moves 1 KiB (1024 / (2 BK) rows) straight from memory into LDS.
template <int ROWS, int BK, int NW>
struct DmaOperand {
    static constexpr int KCH = BK / 8;
    static constexpr int ROWS_PER_KB = 1024 / (2 * BK);
    static constexpr int NB = ROWS / ROWS_PER_KB / NW;  // direct loads per wave per stage
    static_assert(NB * NW * ROWS_PER_KB == ROWS, "DMA split");
    __amdgpu_buffer_rsrc_t rs;
    const uint16_t *base;  // first row of the tile
    int64_t ld, row0, nrows, P;
    uint32_t off[NB];

    __device__ __forceinline__ void init(const uint16_t *g, int64_t ld_, int64_t row0_,
                                         int64_t nrows_, int64_t P_, int wave, int lane)
    {
        ld = ld_, row0 = row0_, nrows = nrows_, P = P_;
        base = g + row0 * ld;
        rs = tile_rsrc(base);
        // Lane l of block b lands at byte 16 l: tile row ROWS_PER_KB*b + l/KCH,
        // LDS slot l%KCH, which holds chunk (l%KCH) ^ swz(row).  Rows past the
        // edge read the last valid row (never stored).
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int row = (wave * NB + i) * ROWS_PER_KB + lane / KCH;
            const int64_t gr = min(row0 + row, nrows - 1) - row0;
            const int kc = (lane % KCH) ^ lds_swz<BK>(row);
            off[i] = static_cast<uint32_t>((gr * ld + kc * 8) * 2);
        }
    }
    __device__ __forceinline__ void dma(uint16_t *lds, int64_t p0, int wave)
    {
#pragma unroll
        for (int i = 0; i < NB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, LMH_LDS_PTR(lds + (wave * NB + i) * 512), 16, static_cast<int>(off[i]),
                static_cast<int>(p0 * 2), 0, 0);
    }
    // Guarded register path (ragged tail stage, edge tiles): zero past P.
    template <int NT>
    __device__ __forceinline__ void staged(uint16_t *lds, int64_t p0, int tid)
    {
        constexpr int RSTEP = NT / KCH;
        const int crow = tid / KCH, ccol = tid % KCH;
        const int64_t gp = p0 + ccol * 8;
#pragma unroll
        for (int i = 0; i < ROWS / RSTEP; ++i) {
            const int row = crow + i * RSTEP;
            const uint16_t *src = base + (min(row0 + row, nrows - 1) - row0) * ld + gp;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (gp + 8 <= P)
                v = load16(src);
            else if (gp < P)
                v = load_partial(src, static_cast<int>(P - gp));
            *reinterpret_cast<uint4 *>(&lds[row * BK + ((ccol ^ lds_swz<BK>(row)) * 8)]) = v;
        }
    }
};

// An operand stored [P][rows] (rows contiguous), moved into LDS as it lies
// in memory by direct buffer loads: stage layout [BK p-rows][ROWS] BF16, the
// 16-byte chunk c of p-row p kept at chunk c ^ tr_swz(p).  MFMA fragments (8
// consecutive p of one tile row per lane) come from two transposing LDS reads
// (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte reads of lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
// So lane 4b + a of a group addresses p-row p0 + b, tile rows n0 + 4a ..
// n0 + 4a + 3, and lane i then holds tile row n0 + i at p-rows p0 .. p0 + 3.
// With tr_swz(p) = 4 (p % 4) the four p-rows of a group (and two groups
// side by side) read sixteen distinct chunks: no bank conflicts.
__device__ __forceinline__ int tr_swz(int prow)
{
    return (prow & 3) << 2;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

template <int ROWS, int BK, int NW>
struct TrOperand {
    static constexpr int CPR = ROWS / 8;             // 16-byte chunks per p-row
    static constexpr int PPK = 1024 / (2 * ROWS);    // p-rows per 1 KiB direct load
    static constexpr int NB = BK / PPK / NW;         // direct loads per wave per stage
    static_assert(ROWS == 128 || ROWS == 256, "chunk swizzle needs >= 16 chunks per p-row");
    static_assert(NB * NW * PPK == BK, "direct-load split");
    const uint16_t *base;  // element (p = 0, first tile row)
    int64_t ld, row0, nrows, P;
    uint32_t off[NB];
    int fa0[4];  // per-lane byte offset of fragment i's first read (k step 0)

    __device__ __forceinline__ void init(const uint16_t *g, int64_t ld_, int64_t row0_,
                                         int64_t nrows_, int64_t P_, int wave, int lane,
                                         int frow0)
    {
        ld = ld_, row0 = row0_, nrows = nrows_, P = P_;
        base = g + row0;
        // Lane l of block b lands at byte 16 l: p-row PPK*b + l/CPR, LDS chunk
        // l%CPR, which holds the tile's chunk (l%CPR) ^ tr_swz(p-row).
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int prow = (wave * NB + i) * PPK + lane / CPR;
            const int gc = (lane % CPR) ^ tr_swz(prow);
            off[i] = static_cast<uint32_t>((static_cast<int64_t>(prow) * ld + gc * 8) * 2);
        }
        // Fragment reads: lane = 16 g + 4 b + a reads p-row 8 (g / 2) + b (+ 16 kk
        // + 4 h) at tile row frow0 + 32 i + 16 (g % 2) + 4 a.
        const int gq = lane >> 4, b = (lane >> 2) & 3, a = lane & 3;
        const int prow = 8 * (gq >> 1) + b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = frow0 + 32 * i + 16 * (gq & 1) + 4 * a;
            fa0[i] = prow * ROWS * 2 + (((col >> 3) ^ tr_swz(prow)) << 4) + (col & 7) * 2;
        }
    }
    __device__ __forceinline__ void dma(uint16_t *lds, int64_t p0, int wave)
    {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base + p0 * ld);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, LMH_LDS_PTR(lds + (wave * NB + i) * 512), 16, static_cast<int>(off[i]), 0, 0, 0);
    }
    // Guarded register path (ragged p tail, edge tiles): zeros past P and past
    // the last row.
    template <int NT>
    __device__ __forceinline__ void staged(uint16_t *lds, int64_t p0, int tid)
    {
        for (int idx = tid; idx < BK * CPR; idx += NT) {
            const int prow = idx / CPR, c = idx % CPR;
            const int64_t pp = p0 + prow, r = row0 + c * 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (pp < P) {
                const uint16_t *src = base + pp * ld + c * 8;
                if (r + 8 <= nrows)
                    v = load16(src);
                else if (r < nrows)
                    v = load_partial(src, static_cast<int>(nrows - r));
            }
            *reinterpret_cast<uint4 *>(&lds[prow * ROWS + ((c ^ tr_swz(prow)) * 8)]) = v;
        }
    }
    // Fragment i (tile rows frow0 + 32 i ..) of k step kk: 8 consecutive p per lane.
    __device__ __forceinline__ bf16x8 frag(const uint16_t *lds, int i, int kk) const
    {
        typedef __attribute__((address_space(3))) v4i16 lds_v4;
        const char *b0 = reinterpret_cast<const char *>(lds) + fa0[i] + 16 * kk * ROWS * 2;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4 *)(b0));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4 *)(b0 + 4 * ROWS * 2));
        const v8i16 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, c);
    }
};

// Epilogue through LDS: the tile is written out in rounds.  In round t every
// wave puts fragment column t of its accumulators (32 output rows c) into the
// staging buffer of its wave column (stage, and stage2 when WC == 2: the first
// LDS stage buffers, free once the main loop is done), a [32][BR] array with
// 16-byte chunk k of row c stored at chunk k ^ (c % 16) so that both the
// fragment writes and the row reads below hit distinct banks.  Then every wave
// reads whole rows and stores them with one 16-byte access per lane (the MFMA
// result's register layout would store 32 bytes into each of 32 rows per
// instruction; the stores are nontemporal unless g.stream_out is off).  EPI:
// FP32 store, FP32 accumulate (D += tile), or BF16 store
// (rounded to nearest-even in registers by v_cvt_pk_bf16_f32 and staged as
// BF16, 8 values per lane and store).  Every thread of the workgroup must call
// this.
template <int FR, int FC, int WR, int WC, int BR, int BC, int EPI>
__device__ __forceinline__ void store_tile_lds(const GemmProblem &g, f32x16 (&acc)[FR][FC],
                                               int64_t r0, int64_t c0, int wr, int wc, int lane,
                                               int wave, void *stage, void *stage2)
{
    constexpr int TR = FR * 32, TC = FC * 32, NW = WR * WC;
    constexpr bool BF = EPI == static_cast<int>(Epi::kStoreBF16);
    constexpr int ESZ = BF ? 2 : 4;        // bytes per staged element
    constexpr int ROWB = BR * ESZ;         // bytes per staged row
    constexpr int EPC = 16 / ESZ;          // elements per 16-byte chunk
    constexpr int LPR = BR / EPC;          // lanes per row
    constexpr int RPI = 64 / LPR;          // rows per wave instruction
    constexpr int ROWS = 32 * WC;          // rows staged per round
    static_assert(BR == 128 || BR == 256, "staging written for 128- or 256-row tiles");
    static_assert(WC == 1 || WC == 2, "one staging buffer per wave column");
    static_assert(TR * WR == BR && TC * WC == BC, "tile shape");
    static_assert(ROWS % (NW * RPI) == 0, "whole passes");
    char *const sb0 = static_cast<char *>(stage);
    char *const sb1 = static_cast<char *>(WC == 2 ? stage2 : stage);
    char *const own = wc ? sb1 : sb0;
    const int cl = lane & 31;
    __syncthreads();  // every wave is done reading the main loop's stages
#pragma unroll
    for (int t = 0; t < FC; ++t) {
#pragma unroll
        for (int i = 0; i < FR; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rl = wr * TR + i * 32 + q * 8 + (lane >> 5) * 4;  // 4 rows from rl
                if constexpr (BF) {
                    const f32x2 lo = {acc[i][t][4 * q + 0], acc[i][t][4 * q + 1]};
                    const f32x2 hi = {acc[i][t][4 * q + 2], acc[i][t][4 * q + 3]};
                    uint2 w;
                    w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
                    w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
                    *reinterpret_cast<uint2 *>(own + cl * ROWB + (((rl >> 3) ^ (cl & 15)) << 4) +
                                               ((rl >> 2) & 1) * 8) = w;
                } else {
                    float4 v;
                    v.x = acc[i][t][4 * q + 0];
                    v.y = acc[i][t][4 * q + 1];
                    v.z = acc[i][t][4 * q + 2];
                    v.w = acc[i][t][4 * q + 3];
                    *reinterpret_cast<float4 *>(own + cl * ROWB + (((rl >> 2) ^ (cl & 15)) << 4)) =
                        v;
                }
            }
        __syncthreads();
#pragma unroll
        for (int rr0 = 0; rr0 < ROWS; rr0 += NW * RPI) {
            const int rr = rr0 + wave * RPI + lane / LPR;
            const int b = rr >> 5, cs = rr & 31;
            const int k = lane % LPR;
            const int64_t c = c0 + b * TC + t * 32 + cs;
            const int64_t r = r0 + EPC * k;
            const char *src = (b ? sb1 : sb0) + cs * ROWB + ((k ^ (cs & 15)) << 4);
            if (c < g.C && r < g.R) {
                if constexpr (BF) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(src);
                    uint16_t *out = static_cast<uint16_t *>(g.D) + c * g.ldd + r;
                    if (r + 8 <= g.R) {
                        store16(out, v, g.stream_out);
                    } else {
                        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
                        for (int e = 0; e < 8 && r + e < g.R; ++e)
                            out[e] = static_cast<uint16_t>(vv[e >> 1] >> (16 * (e & 1)));
                    }
                } else {
                    const float4 v = *reinterpret_cast<const float4 *>(src);
                    float *out = static_cast<float *>(g.D) + c * g.ldd + r;
                    if (r + 4 <= g.R) {
                        float4 w = v;
                        if constexpr (EPI == static_cast<int>(Epi::kAccumF32)) {
                            const float4 o = *reinterpret_cast<const float4 *>(out);
                            w.x += o.x, w.y += o.y, w.z += o.z, w.w += o.w;
                        }
                        store16(out, w, g.stream_out);
                    } else {
                        const float vv[4] = {v.x, v.y, v.z, v.w};
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
        __syncthreads();
    }
}

// Cross-entropy partial statistics of a finished logits tile, from the FP32
// accumulators just stored (R = vocabulary, C = tokens; the tile covers
// vocabulary rows [r0, r0 + WR * 32 FR) and tokens [c0, c0 + BC)).  For every
// token the record {m, d, X_y, own} of the tile's vocabulary block: m = max,
// d = sum exp(z - m) over the block's rows below R, X_y = the stored logit of
// the token's target row when it lies in the block (own = 1), else 0 and 0.
// Lane l holds rows wr*TR + 32 i + 8 q + 4 (l / 32) + e (i < FR, q, e < 4) of
// its FC tokens; lanes l and l ^ 32 hold the two halves of the wave's rows;
// the WR waves along the rows are combined in order through LDS.  yt[j] is
// the target of the lane's token j (loaded before the tile's stores).  Every
// thread of the workgroup must call this (one barrier).
template <int FR, int FC>
__device__ __forceinline__ void tile_targets(const GemmProblem &g, int64_t c0, int wc, int lane,
                                             int32_t (&yt)[FC])
{
#pragma unroll
    for (int j = 0; j < FC; ++j) {
        const int64_t c = c0 + wc * FC * 32 + j * 32 + (lane & 31);
        yt[j] = (c < g.C) ? g.tgt[c] : g.ignore_index;
    }
}

template <int FR, int FC, int WR, int BC>
__device__ __forceinline__ void stats_tile(const GemmProblem &g, f32x16 (&acc)[FR][FC],
                                           const int32_t (&yt)[FC], int64_t r0, int64_t c0,
                                           int64_t tile_r, int wr, int wc, int lane, int tid)
{
    constexpr int TR = FR * 32, TC = FC * 32;
    __shared__ float4 ep[WR][BC];
    const int64_t rw = r0 + wr * TR;  // the wave's first row
    const int half = lane >> 5;
    const bool interior = rw + TR <= g.R;
#pragma unroll
    for (int j = 0; j < FC; ++j) {
        const int tok = wc * TC + j * 32 + (lane & 31);
        // The target's position in this wave's rows, if it is one of this lane's.
        const int64_t lr64 = static_cast<int64_t>(yt[j]) - rw;
        const bool mine = yt[j] != g.ignore_index && lr64 >= 0 && lr64 < TR &&
                          ((lr64 >> 2) & 1) == half;
        const int lr = mine ? static_cast<int>(lr64) : -1;
        const int ti = lr >> 5, tq = (lr >> 3) & 3, te = lr & 3;
        float m = -INFINITY, d = 0.0f, x = 0.0f;
        if (interior) {
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    m = fmaxf(m, acc[i][j][e]);
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    d += exp_shifted(acc[i][j][e], m);
        } else {
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (rw + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3) < g.R)
                        m = fmaxf(m, acc[i][j][e]);
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (rw + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3) < g.R)
                        d += exp_shifted(acc[i][j][e], m);
        }
#pragma unroll
        for (int i = 0; i < FR; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                x = (i == ti && (e >> 2) == tq && (e & 3) == te) ? acc[i][j][e] : x;
        const float own = mine ? 1.0f : 0.0f;
        const float m2 = __shfl_xor(m, 32, 64), d2 = __shfl_xor(d, 32, 64);
        const float x2 = __shfl_xor(x, 32, 64), own2 = __shfl_xor(own, 32, 64);
        merge_md(m, d, m2, d2);
        if (lane < 32)
            ep[wr][tok] = make_float4(m, d, mine ? x : x2, own + own2);
    }
    __syncthreads();
    for (int tok = tid; tok < BC; tok += WR * (BC / TC) * 64) {
        const int64_t c = c0 + tok;
        if (c >= g.C)
            continue;
        float4 rec = ep[0][tok];
        for (int w = 1; w < WR; ++w) {
            const float4 q = ep[w][tok];
            merge_md(rec.x, rec.y, q.x, q.y);
            if (q.w != 0.0f) {
                rec.z = q.z;
                rec.w += q.w;
            }
        }
        static_cast<float4 *>(g.part4)[tile_r * g.part_stride4 + c] = rec;
    }
}

// ---------------------------------------------------------------------------
// gemm_big: BR x BC tiles, WR x WC waves (two per SIMD with 8 waves), BK = 64.
// Both operands stream into LDS by direct buffer loads.  An operand whose
// contraction dimension is contiguous (the logits' x and W, dgrad's dlogits)
// is stored k-contiguous per tile row; a p-major one (dgrad's W, wgrad's x and
// dlogits) is stored as it lies in memory, p-rows of the tile's row range,
// and its MFMA fragments are read with transposing LDS loads
// (ds_read_b64_tr_b16), so no register transpose is needed.  Two LDS stages
// per operand as separate arrays, so that the compiler can tell a direct load
// into one stage from the fragment reads of the other (the steady loop is
// unrolled by two to keep the stage choice compile-time).
//
// Steady state (interior tile, full stages), per stage kt:
//   top:   direct loads of stage kt+1 into the other stage (spread over the
//          first 16-wide k step, one per MFMA);
//   k0-2:  fragment reads one k step ahead of the MFMAs;
//   k3:    half the MFMAs, the workgroup barrier (after this wave's direct
//          loads landed), the first fragment reads of stage kt+1, the other
//          half of the MFMAs -- the barrier and the read latency hide behind
//          matrix work.
// Edge tiles and the last stages run a guarded loop with the same layout.
template <int BR, int BC, int BK, int WR, int WC, bool AT, bool BT, int EPI>
__global__ void __launch_bounds__(WR * WC * 64)
    __attribute__((amdgpu_waves_per_eu(WR * WC / 4, WR * WC / 4)))
gemm_big(GemmProblem gp, TileMap tm)
{
    // Split of the sum over p (blockIdx.y): this workgroup's p range and its
    // FP32 partial tile (see GemmProblem::psplit).
    GemmProblem g = gp;
    if (gp.psplit > 0) {
        const int64_t p0 = min(static_cast<int64_t>(blockIdx.y) * gp.psplit, gp.P);
        g.P = min(gp.psplit, gp.P - p0);
        g.A = gp.A + (AT ? p0 * gp.lda : p0);
        g.B = gp.B + (BT ? p0 * gp.ldb : p0);
        g.D = static_cast<float *>(gp.D) + blockIdx.y * gp.split_stride;
    }
    constexpr int NT = WR * WC * 64;
    constexpr int NW = WR * WC;
    constexpr int TR = BR / WR, TC = BC / WC;
    constexpr int FR = TR / 32, FC = TC / 32;
    constexpr int NKK = BK / 16;
    static_assert(BK == 64 && NKK == 4 && FR % 2 == 0, "schedule written for BK = 64");
    static_assert(32 * BR * 4 <= BR * BK * 2, "the FP32 epilogue stages 32 rows in sA0, sA1");
    // p-major operands (AT / BT) are read through transposing LDS loads.
    using OpA = std::conditional_t<AT, TrOperand<BR, BK, NW>, DmaOperand<BR, BK, NW>>;
    using OpB = std::conditional_t<BT, TrOperand<BC, BK, NW>, DmaOperand<BC, BK, NW>>;

    __shared__ __attribute__((aligned(16))) uint16_t sA0[BR * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA1[BR * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB0[BC * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB1[BC * BK];

    int tr, tc;
    map_tile(tm, tr, tc);
    const int64_t r0 = static_cast<int64_t>(tr) * BR;
    const int64_t c0 = static_cast<int64_t>(tc) * BC;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wr = wave % WR;
    const int wc = wave / WR;
    // Direct-load operands clamp rows past the edge (those outputs are never
    // stored); only transposed operands need the tile inside the rows.
    const bool interior = (!AT || r0 + BR <= g.R) && (!BT || c0 + BC <= g.C);

    OpA opA;
    OpB opB;
    if constexpr (AT)
        opA.init(g.A, g.lda, r0, g.R, g.P, wave, lane, wr * TR);
    else
        opA.init(g.A, g.lda, r0, g.R, g.P, wave, lane);
    if constexpr (BT)
        opB.init(g.B, g.ldb, c0, g.C, g.P, wave, lane, wc * TC);
    else
        opB.init(g.B, g.ldb, c0, g.C, g.P, wave, lane);

    // Per-lane fragment addressing.  Fragment i of a wave covers tile rows
    // wr*TR + 32i + (lane%32); the XOR key of its chunk index (lane/32 is the
    // lane's half of the 16-wide k step) depends on i only through its parity.
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const int fbA = (wr * TR + lrow) * BK;
    const int fbB = (wc * TC + lrow) * BK;
    int keyA[2], keyB[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        keyA[par] = khalf ^ lds_swz<BK>(wr * TR + par * 32 + lrow);
        keyB[par] = khalf ^ lds_swz<BK>(wc * TC + par * 32 + lrow);
    }
    bf16x8 fa[2][FR], fb[2][FC];
    auto frag_load = [&](const uint16_t *lA, const uint16_t *lB, int kk, int slot) {
        const int ka0 = ((2 * kk) ^ keyA[0]) * 8, ka1 = ((2 * kk) ^ keyA[1]) * 8;
        const int kb0 = ((2 * kk) ^ keyB[0]) * 8, kb1 = ((2 * kk) ^ keyB[1]) * 8;
#pragma unroll
        for (int i = 0; i < FR; ++i) {
            if constexpr (AT)
                fa[slot][i] = opA.frag(lA, i, kk);
            else
                fa[slot][i] = *reinterpret_cast<const bf16x8 *>(
                    &lA[fbA + i * 32 * BK + ((i & 1) ? ka1 : ka0)]);
        }
#pragma unroll
        for (int j = 0; j < FC; ++j) {
            if constexpr (BT)
                fb[slot][j] = opB.frag(lB, j, kk);
            else
                fb[slot][j] = *reinterpret_cast<const bf16x8 *>(
                    &lB[fbB + j * 32 * BK + ((j & 1) ? kb1 : kb0)]);
        }
    };

    f32x16 acc[FR][FC];
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FC; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;
    auto mfma_rows = [&](int slot, int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < FC; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j],
                                                                    acc[i][j], 0, 0, 0);
    };
    auto compute_stage = [&](const uint16_t *lA, const uint16_t *lB) {
        frag_load(lA, lB, 1, 1);
        mfma_rows(0, 0, FR);
        frag_load(lA, lB, 2, 0);
        mfma_rows(1, 0, FR);
        frag_load(lA, lB, 3, 1);
        mfma_rows(0, 0, FR);
        mfma_rows(1, 0, FR);
    };

    // One steady-state stage (see the comment above the kernel).
    auto stage_fast = [&](const uint16_t *cA, const uint16_t *cB, uint16_t *nA, uint16_t *nB,
                          int64_t kt) {
        constexpr int nmf = FR * FC;
        constexpr int nrd = FR * (AT ? 2 : 1) + FC * (BT ? 2 : 1);  // LDS reads per k step
        constexpr int ndma = OpA::NB + OpB::NB;
        opA.dma(nA, (kt + 1) * BK, wave);
        opB.dma(nB, (kt + 1) * BK, wave);
        frag_load(cA, cB, 1, 1);
        mfma_rows(0, 0, FR);
        frag_load(cA, cB, 2, 0);
        mfma_rows(1, 0, FR);
        frag_load(cA, cB, 3, 1);
        mfma_rows(0, 0, FR);
        mfma_rows(1, 0, FR / 2);
        // Interleave of k steps 0-2: their MFMAs, the next step's fragment
        // reads, and (step 0) the direct loads of stage kt+1.
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
            for (int m = 0; m < nmf; ++m) {
                if (s == 0 && m < ndma)
                    __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                if (m < nrd)
                    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(kSgMfma, nmf / 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        // This wave's direct loads of stage kt+1 have landed; then the barrier.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        frag_load(nA, nB, 0, 0);
        mfma_rows(1, FR / 2, FR);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, nrd, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, nmf / 2, 0);
    };

    const int64_t nk = (g.P + BK - 1) / BK;
    const int64_t nfull = g.P / BK;
    int64_t kt = 0;
    // Prologue: stage 0 into stage buffer 0.
    if (nk > 0) {
        const bool fast0 = interior && nfull > 0;
        if (fast0) {
            opA.dma(sA0, 0, wave);
            opB.dma(sB0, 0, wave);
        } else {
            opA.template staged<NT>(sA0, 0, tid);
            opB.template staged<NT>(sB0, 0, tid);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        frag_load(sA0, sB0, 0, 0);
    }
    if (interior) {
        for (; kt + 3 <= nfull; kt += 2) {
            stage_fast(sA0, sB0, sA1, sB1, kt);
            stage_fast(sA1, sB1, sA0, sB0, kt + 1);
        }
        // One more (stage kt is in buffer 0) when the next stage is full, so
        // that only the last full stage is computed without a load behind it.
        if (kt + 1 < nfull) {
            stage_fast(sA0, sB0, sA1, sB1, kt);
            ++kt;
        }
    }
    // Remaining stages (all of them for an edge tile): guarded register loads
    // with zero fill.  On entry, stage kt is in stage buffer kt&1 with its
    // first fragments read.
    for (; kt < nk; ++kt) {
        uint16_t *cA = (kt & 1) ? sA1 : sA0;
        uint16_t *cB = (kt & 1) ? sB1 : sB0;
        uint16_t *nA = (kt & 1) ? sA0 : sA1;
        uint16_t *nB = (kt & 1) ? sB0 : sB1;
        compute_stage(cA, cB);
        if (kt + 1 < nk) {
            opA.template staged<NT>(nA, (kt + 1) * BK, tid);
            opB.template staged<NT>(nB, (kt + 1) * BK, tid);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + 1 < nk)
            frag_load(nA, nB, 0, 0);
    }

    if constexpr (EPI == static_cast<int>(Epi::kStoreF32Stats) && !AT && !BT) {
        int32_t yt[FC];
        tile_targets<FR, FC>(g, c0, wc, lane, yt);  // in flight during the stores
        store_tile_lds<FR, FC, WR, WC, BR, BC, 0>(g, acc, r0, c0, wr, wc, lane, wave, sA0, sA1);
        stats_tile<FR, FC, WR, BC>(g, acc, yt, r0, c0, tr, wr, wc, lane, tid);
    } else {
        store_tile_lds<FR, FC, WR, WC, BR, BC, EPI>(g, acc, r0, c0, wr, wc, lane, wave, sA0,
                                                     sA1);
    }
}

// ---------------------------------------------------------------------------
// gemm_small: the logits GEMM for few tokens (M <= 256), where the work is
// bound by streaming W once from HBM.  Tiles of 128 vocabulary rows x BC
// tokens (BC = 32, 64, 128 or 256), 4 waves (each 32 rows x BC), BK = 64, and a
// ring of S LDS stages filled by direct buffer loads: S-1 stages are in
// flight while one is consumed, which keeps enough bytes moving per CU to
// approach the HBM rate.  The steady loop is unrolled S times so that every
// stage buffer is a compile-time choice (the compiler then knows the loads
// in flight never touch the buffer being read).
template <int... I, typename F>
__device__ __forceinline__ void unroll_seq(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>{}), ...);
}

// One LDS array per (TAG, size): distinct variables let the compiler prove
// that a direct load into one ring stage never touches another.
template <int TAG, int N>
__device__ __forceinline__ uint16_t *lds_array()
{
    __shared__ __attribute__((aligned(16))) uint16_t buf[N];
    return buf;
}

template <int BC, int S, int EPI, int BK>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_small(GemmProblem g, TileMap tm)
{
    constexpr int BR = 128, NW = 4;
    constexpr int FR = 1, FC = BC / 32;
    using OpA = DmaOperand<BR, BK, NW>;
    using OpB = DmaOperand<BC, BK, NW>;
    constexpr int NBW = OpA::NB + OpB::NB;  // direct loads per wave per stage
    static_assert(S >= 3, "ring of at least three stages");

    // Stage buffers: sA(b) / sB(b) for a compile-time b, and tables for the
    // runtime-indexed tail.
    auto sA_c = [](auto bc) { return lds_array<2 * decltype(bc)::value, BR * BK>(); };
    auto sB_c = [](auto bc) { return lds_array<2 * decltype(bc)::value + 1, BC * BK>(); };
    uint16_t *sA[S];
    uint16_t *sB[S];
    unroll_seq(std::make_integer_sequence<int, S>{}, [&](auto bc) {
        sA[decltype(bc)::value] = sA_c(bc);
        sB[decltype(bc)::value] = sB_c(bc);
    });

    int tr, tc;
    map_tile(tm, tr, tc);
    const int64_t r0 = static_cast<int64_t>(tr) * BR;
    const int64_t c0 = static_cast<int64_t>(tc) * BC;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    OpA opA;
    OpB opB;
    opA.init(g.A, g.lda, r0, g.R, g.P, wave, lane);
    opB.init(g.B, g.ldb, c0, g.C, g.P, wave, lane);

    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const int fbA = (wave * 32 + lrow) * BK;
    const int fbB = lrow * BK;
    const int keyA = khalf ^ lds_swz<BK>(wave * 32 + lrow);
    int keyB[FC];
#pragma unroll
    for (int j = 0; j < FC; ++j)
        keyB[j] = khalf ^ lds_swz<BK>(j * 32 + lrow);

    f32x16 acc[FR][FC];
#pragma unroll
    for (int j = 0; j < FC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[0][j][e] = 0.0f;

    auto compute = [&](const uint16_t *lA, const uint16_t *lB) {
        bf16x8 fa[2], fb[2][FC];
        auto fl = [&](int kk, int slot) {
            fa[slot] = *reinterpret_cast<const bf16x8 *>(&lA[fbA + (((2 * kk) ^ keyA) * 8)]);
#pragma unroll
            for (int j = 0; j < FC; ++j)
                fb[slot][j] = *reinterpret_cast<const bf16x8 *>(
                    &lB[fbB + j * 32 * BK + ((2 * kk) ^ keyB[j]) * 8]);
        };
        fl(0, 0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            if (kk + 1 < BK / 16)
                fl(kk + 1, (kk + 1) & 1);
#pragma unroll
            for (int j = 0; j < FC; ++j)
                acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1], fb[kk & 1][j],
                                                                    acc[0][j], 0, 0, 0);
        }
    };

    const int64_t nk = (g.P + BK - 1) / BK;
    const int64_t nfull = g.P / BK;
    // Stage s reads k block (s + rot) mod nk, rot = the tile row mod nk (all
    // stages full only; a ragged last stage keeps the plain order).  Every
    // tile streams its W rows over the same k block at once otherwise, and
    // with a row pitch of 16 KiB those requests pile onto few HBM channels;
    // staggering the start spreads them.  Tiles that share W rows (same tile
    // row) stay in step, so their L2 sharing is kept.  Measured on MI355X,
    // V=32768: M=32 K=8192 100.7 -> 89.2 us, M=64 104.3 -> 91.5, M=128
    // 141.6 -> 129.0, K=16384 -2 %, K=1024 -4 %, others within 1 %.
    const int64_t rot = nk == nfull && nk > 0 ? static_cast<int64_t>(tr) % nk : 0;
    auto pk = [&](int64_t st) {
        const int64_t q = st + rot;
        return (q >= nk ? q - nk : q) * BK;
    };
    // Prologue: the first S-1 full stages go in flight.
    unroll_seq(std::make_integer_sequence<int, S - 1>{}, [&](auto bc) {
        constexpr int st = decltype(bc)::value;
        if (st < nfull) {
            opA.dma(sA_c(bc), pk(st), wave);
            opB.dma(sB_c(bc), pk(st), wave);
        }
    });
    int64_t kt = 0;
    // Steady state: S consecutive stages per trip, each waiting only for its
    // own loads (the S-2 later stages stay in flight), then refilling the
    // buffer freed by the previous stage.
    for (; kt + 2 * S - 2 < nfull; kt += S) {
        unroll_seq(std::make_integer_sequence<int, S>{}, [&](auto bc) {
            constexpr int b = decltype(bc)::value;
            constexpr int bn = (b + S - 1) % S;
            constexpr int outstanding = (S - 2) * NBW;
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(outstanding) : "memory");
            const int64_t pn = pk(kt + b + S - 1);
            const std::integral_constant<int, bn> bnc;
            opA.dma(sA_c(bnc), pn, wave);
            opB.dma(sB_c(bnc), pn, wave);
            compute(sA_c(bc), sB_c(bc));
        });
    }
    // Remaining stages: conservative waits; a ragged last stage is loaded
    // through registers with zero fill past P.
    for (; kt < nk; ++kt) {
        const int b = static_cast<int>(kt % S);
        if (kt >= nfull) {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            opA.template staged<256>(sA[b], kt * BK, tid);
            opB.template staged<256>(sB[b], kt * BK, tid);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + S - 1 < nfull) {
            const int bn = static_cast<int>((kt + S - 1) % S);
            opA.dma(sA[bn], pk(kt + S - 1), wave);
            opB.dma(sB[bn], pk(kt + S - 1), wave);
        }
        compute(sA[b], sB[b]);
    }
    store_tile_lds<FR, FC, NW, 1, BR, BC, EPI>(g, acc, r0, c0, wave, 0, lane, wave,
                                               sA_c(std::integral_constant<int, 0>{}), nullptr);
}

template <int BC, int S, int BK = 64>
hipError_t launch_small(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    TileMap tm;
    tm.tiles_r = static_cast<int>((p.R + 127) / 128);
    tm.tiles_c = static_cast<int>((p.C + BC - 1) / BC);
    tm.group_r = std::min(std::max(group_r, 1), std::max(tm.tiles_r, 1));
    const int64_t nwg = static_cast<int64_t>(tm.tiles_r) * tm.tiles_c;
    if (nwg == 0)
        return hipSuccess;
    if (epi == Epi::kStoreBF16)
        hipLaunchKernelGGL((gemm_small<BC, S, 1, BK>), dim3(static_cast<unsigned>(nwg)), dim3(256), 0,
                           s, p, tm);
    else
        hipLaunchKernelGGL((gemm_small<BC, S, 0, BK>), dim3(static_cast<unsigned>(nwg)), dim3(256), 0,
                           s, p, tm);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gemm_pp: the logits GEMM for many tokens (both operands K-contiguous,
// K a multiple of 32).  256 x 256 tiles, 8 waves of 64 x 128 accumulators,
// K consumed in stages of 32 held in a ring of four LDS slots that direct
// buffer loads fill three stages ahead.
//
// The waves form two groups (waves 0-3 and 4-7, one of each per SIMD) that
// run the same sequence, one phase apart ("ping-pong"):
//   M(s): issue this wave's direct loads of stage s+3, read its stage-s
//         fragments (two 16-wide k steps) into registers, wait for its loads
//         of stage s+1; barrier;
//   C(s): the 16 MFMAs of stage s from registers; barrier.
// Group 1 enters with one extra barrier, so while one group issues its 16
// back-to-back MFMAs the other group on the same SIMD does its memory work
// and waits; the matrix pipe changes hands at every barrier instead of
// idling through the waits.  Every wave executes 2N + 2 barriers (N stages).
// Ring safety, with barriers numbered per group: stage s+3 overwrites the
// slot of stage s-1, whose reads both groups finished (lgkmcnt(0)) before
// barriers that precede either group's M(s); each wave waits for its own
// loads of stage s+1 before the barrier that ends its M(s), and both groups'
// waits precede the barrier after which group 0 runs M(s+1).
//
// LDS slot layout per operand: [256 rows][32] BF16 (64-byte rows); the four
// 16-byte chunks of a row are permuted by pp_swz(row), which keeps both the
// 1 KiB direct-load blocks and the MFMA fragment reads free of bank
// conflicts whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int pp_swz(int row)
{
    return ((row >> 1) & 3) ^ ((row >> 3) & 1);
}

// Wait until at most N of this wave's direct loads are in flight.  Inline
// assembly, like the loads themselves: the compiler neither sees nor adds to
// the waits of the ring.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LMH_LDS_PTR(p)));
}

// One 16-byte-per-lane direct load into LDS at lds + 16 * lane, issued from
// inline assembly so that the compiler does not track it: the kernel's own
// vmcnt waits and barriers order every use of the destination.  M0 holds the
// LDS base (an input operand, so the compiler writes it); one wait state
// separates that write from the load.
__device__ __forceinline__ void dma16_untracked(__amdgpu_buffer_rsrc_t rs, uint32_t lds,
                                                uint32_t voff, int soff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

__device__ __forceinline__ void pp_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int EPI>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_pp(GemmProblem g, TileMap tm)
{
    constexpr int BR = 256, BC = 256, BK = 32, S = 4;
    constexpr int WR = 4, TR = 64, TC = 128, FR = TR / 32, FC = TC / 32;
    constexpr int SLOT = 256 * BK;  // BF16 elements per operand per slot (16 KiB)
    // One LDS array per slot (A then B): the compiler tracks only a few
    // direct-load targets; beyond that it waits for every load in flight.
    constexpr int TAG = 64;
    auto sA = [](auto bc) { return lds_array<TAG + decltype(bc)::value, 2 * SLOT>(); };
    auto sB = [](auto bc) { return lds_array<TAG + decltype(bc)::value, 2 * SLOT>() + SLOT; };

    int tr, tc;
    map_tile(tm, tr, tc);
    const int64_t r0 = static_cast<int64_t>(tr) * BR;
    const int64_t c0 = static_cast<int64_t>(tc) * BC;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WR;
    const int grp = wave / WR;  // also the tile's column half

    // Direct loads: this wave moves rows [32 wave, 32 wave + 32) of both
    // operand tiles, as two 1 KiB blocks of 16 rows; lane l lands at byte 16 l
    // of its block (row l/4, slot l%4) and fetches chunk (l%4) ^ pp_swz(row).
    // Rows past the edge re-read the last valid row (never stored).
    const __amdgpu_buffer_rsrc_t rsA = tile_rsrc(g.A + r0 * g.lda);
    const __amdgpu_buffer_rsrc_t rsB = tile_rsrc(g.B + c0 * g.ldb);
    uint32_t offA[2], offB[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int row = 32 * wave + 16 * b + lane / 4;
        const int ch = (lane & 3) ^ pp_swz(row);
        offA[b] = static_cast<uint32_t>(((min(r0 + row, g.R - 1) - r0) * g.lda + ch * 8) * 2);
        offB[b] = static_cast<uint32_t>(((min(c0 + row, g.C - 1) - c0) * g.ldb + ch * 8) * 2);
    }
    auto dma = [&](uint16_t *lA, uint16_t *lB, int64_t st) {
        const int soff = static_cast<int>(st * BK * 2);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            dma16_untracked(rsA, lds_addr(lA + (2 * wave + b) * 512), offA[b], soff);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            dma16_untracked(rsB, lds_addr(lB + (2 * wave + b) * 512), offB[b], soff);
    };

    // Fragment reads: fragment i of the wave covers tile rows wr*TR + 32i +
    // lane%32; pp_swz of those rows depends on lane%32 only.
    const int key = pp_swz(lane & 31);
    const int hk = lane >> 5;
    const int fbA = (wr * TR + (lane & 31)) * BK;
    const int fbB = (grp * TC + (lane & 31)) * BK;
    bf16x8 fa[2][FR], fb[2][FC];
    auto frag_read = [&](const uint16_t *lA, const uint16_t *lB) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ch = ((2 * kk + hk) ^ key) * 8;
#pragma unroll
            for (int i = 0; i < FR; ++i)
                fa[kk][i] = *reinterpret_cast<const bf16x8 *>(&lA[fbA + i * 32 * BK + ch]);
#pragma unroll
            for (int j = 0; j < FC; ++j)
                fb[kk][j] = *reinterpret_cast<const bf16x8 *>(&lB[fbB + j * 32 * BK + ch]);
        }
    };

    f32x16 acc[FR][FC];
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FC; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    const int64_t N = g.P / BK;
    // One stage: M(s) then C(s).  SL = s % S is a compile-time slot; FULL
    // (s + 3 < N known) drops the run-time checks of the steady loop.
    auto stage = [&](auto slc, auto fullc, int64_t st) {
        constexpr int SL = decltype(slc)::value;
        constexpr bool FULL = decltype(fullc)::value;
        const std::integral_constant<int, (SL + S - 1) % S> nxc;
        if (FULL || st + 3 < N)
            dma(sA(nxc), sB(nxc), st + 3);
        frag_read(sA(slc), sB(slc));
        // This wave's loads of stage st+1 have landed once at most the
        // groups issued after them (stages st+2, st+3) are outstanding.
        if (FULL || st + 3 < N)
            vm_wait<8>();
        else if (st + 2 < N)
            vm_wait<4>();
        else
            vm_wait<0>();
        pp_barrier();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int j = 0; j < FC; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j],
                                                                        acc[i][j], 0, 0, 0);
        pp_barrier();
    };

    // Prologue: stages 0-2 in flight, wait for stage 0.
    unroll_seq(std::make_integer_sequence<int, S - 1>{}, [&](auto bc) {
        if (decltype(bc)::value < N)
            dma(sA(bc), sB(bc), decltype(bc)::value);
    });
    if (N > 2)
        vm_wait<8>();
    else if (N > 1)
        vm_wait<4>();
    else
        vm_wait<0>();
    pp_barrier();
    if (grp == 1)
        pp_barrier();
    int64_t st = 0;
    const std::true_type full;
    const std::false_type guarded;
    for (; st + S + 3 <= N; st += S)
        unroll_seq(std::make_integer_sequence<int, S>{},
                   [&](auto bc) { stage(bc, full, st + decltype(bc)::value); });
    // The loop leaves st % S == 0 with at most S + 2 stages to go.
    unroll_seq(std::make_integer_sequence<int, S + 2>{}, [&](auto bc) {
        constexpr int k = decltype(bc)::value;
        if (st + k < N)
            stage(std::integral_constant<int, k % S>{}, guarded, st + k);
    });
    if (grp == 0)
        pp_barrier();

    if constexpr (EPI == static_cast<int>(Epi::kStoreF32Stats)) {
        int32_t yt[FC];
        tile_targets<FR, FC>(g, c0, grp, lane, yt);  // in flight during the stores
        store_tile_lds<FR, FC, WR, 2, BR, BC, 0>(g, acc, r0, c0, wr, grp, lane, wave,
                                                 sA(std::integral_constant<int, 0>{}),
                                                 sA(std::integral_constant<int, 1>{}));
        stats_tile<FR, FC, WR, BC>(g, acc, yt, r0, c0, tr, wr, grp, lane, tid);
    } else {
        store_tile_lds<FR, FC, WR, 2, BR, BC, EPI>(g, acc, r0, c0, wr, grp, lane, wave,
                                                   sA(std::integral_constant<int, 0>{}),
                                                   sA(std::integral_constant<int, 1>{}));
    }
}

// ---------------------------------------------------------------------------
// gemm_rows: the logits GEMM for at most 16 tokens, bound by streaming W once
// from HBM.  Reading W as gemm_small does -- every workgroup walking its 128
// rows together in 128-byte steps, so all V rows are open in DRAM at once --
// measured ~4.4 TB/s; reading 32 rows at a time, each over the whole of K in
// 1 KiB steps, ~5.8 TB/s.  So each workgroup (4 waves) takes groups of 32
// vocabulary rows one after another and streams each group over K in stages
// of 512: W [32][512] and the tokens' x [16][512] (tokens past M repeat the
// last one and are never stored) by direct loads into a ring of three stages
// (48 KiB each; with the partial-sum area, all 160 KiB of LDS).  Wave w multiplies k range [128 w, 128 w + 128)
// of every stage (8 MFMAs of 32 x 32 x 16), so the four waves hold partial
// sums of the same 32 x 32 block; after a group's last stage they are added
// through LDS and stored, while the next group's first stages load.  LDS rows
// are 1 KiB; 16-byte chunk c of staged row q sits at chunk c ^ (q % 16), so
// the 16 lanes of a fragment read hit distinct banks.
template <int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_rows(GemmProblem g, int groups_per_wg)
{
    constexpr int XR = 16, S = 3;
    constexpr int RG = 32, BKS = 512;
    constexpr int SLOT = (RG + XR) * BKS;     // BF16 elements per stage (W rows, then x)
    constexpr int NDMA = (RG + XR) / 4;       // direct loads (one staged row each) per wave
    static_assert(S * SLOT * 2 + 4 * 32 * 32 * 4 <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint16_t ring[S * SLOT];
    __shared__ __attribute__((aligned(16))) float red[4][32][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ngroups = (g.R + RG - 1) / RG;
    const int64_t gfirst = static_cast<int64_t>(blockIdx.x) * groups_per_wg;
    const int ng = static_cast<int>(min(static_cast<int64_t>(groups_per_wg), ngroups - gfirst));
    const int nks = static_cast<int>(g.P / BKS);
    const int T = ng * nks;

    // Direct loads of this wave: staged rows q = wave * NDMA + i.  W rows
    // past V and token rows past M repeat the last valid row.
    const __amdgpu_buffer_rsrc_t rsX = tile_rsrc(g.B);
    uint32_t offW[NDMA], offX[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int q = wave * NDMA + i;
        const int sw = q & 15;
        const uint32_t gc = static_cast<uint32_t>(lane ^ sw);  // global chunk of this lane
        offW[i] = static_cast<uint32_t>(q < RG ? (q * g.lda + gc * 8) * 2 : 0);
        const int64_t tok = min(static_cast<int64_t>(q - RG), g.C - 1);
        offX[i] = static_cast<uint32_t>(q >= RG ? (tok * g.ldb + gc * 8) * 2 : 0);
    }
    auto issue = [&](int t) {
        const int gi = t / nks, ks = t - gi * nks;
        const int64_t row0 = (gfirst + gi) * RG;
        const int soff = ks * BKS * 2;
        uint16_t *st = ring + (t % S) * SLOT;
        // W rows of this group past V: clamp the group base so that every
        // row read lies inside W (those rows' results are not stored).
        const int64_t wbase = min(row0, g.R - RG > 0 ? g.R - RG : 0);
        const __amdgpu_buffer_rsrc_t rsW = tile_rsrc(g.A + wbase * g.lda);
        const int rshift = static_cast<int>(row0 - wbase);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int q = wave * NDMA + i;
            if (q < RG) {
                const int qr = min(q + rshift, static_cast<int>(min<int64_t>(g.R - wbase, RG)) - 1);
                const uint32_t off = offW[i] + static_cast<uint32_t>(((qr - q) * g.lda) * 2);
                dma16_untracked(rsW, lds_addr(st + q * BKS), off, soff);
            } else {
                dma16_untracked(rsX, lds_addr(st + q * BKS), offX[i], soff);
            }
        }
    };

    const int lrow = lane & 31, kh = lane >> 5;
    const int xrow = lrow & 15;  // MFMA token columns 16 .. 31 repeat 0 .. 15 (not stored)
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        acc[e] = 0.0f;

    // Prologue: stages 0 .. S-2 in flight.
#pragma unroll
    for (int t = 0; t < S - 1; ++t)
        if (t < T)
            issue(t);
    for (int t = 0; t < T; ++t) {
        // This wave's loads of stage t have landed (stages t+1 .. t+S-2 may
        // still be in flight), then every wave's; the slot of stage t-1 is
        // free once every wave is past this barrier.
        if (t + S - 2 < T)
            vm_wait<(S - 2) * NDMA>();
        else
            vm_wait<0>();
        pp_barrier();
        if (t + S - 1 < T)
            issue(t + S - 1);
        const uint16_t *st = ring + (t % S) * SLOT;
        const uint16_t *sW = st + lrow * BKS;
        const uint16_t *sX = st + (RG + xrow) * BKS;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 16 * wave + 2 * j + kh;  // chunk of k = 128 wave + 16 j + 8 kh
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sW + ((c ^ (lrow & 15)) * 8));
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(sX + ((c ^ ((RG + xrow) & 15)) * 8));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        if ((t + 1) % nks == 0) {
            // Last stage of group gi: add the four waves' partial sums.
            // Lane l holds token l % 32 at rows 8 q + 4 (l / 32) + e.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 v;
                v.x = acc[4 * q + 0];
                v.y = acc[4 * q + 1];
                v.z = acc[4 * q + 2];
                v.w = acc[4 * q + 3];
                *reinterpret_cast<float4 *>(&red[wave][lrow][8 * q + 4 * kh]) = v;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[e] = 0.0f;
            pp_barrier();
            const int c = tid >> 3, r4 = (tid & 7) * 4;
            float4 sum = *reinterpret_cast<const float4 *>(&red[0][c][r4]);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const float4 v = *reinterpret_cast<const float4 *>(&red[w][c][r4]);
                sum.x += v.x, sum.y += v.y, sum.z += v.z, sum.w += v.w;
            }
            const int64_t r = (gfirst + t / nks) * RG + r4;
            if (c < g.C && r < g.R) {
                const float vv[4] = {sum.x, sum.y, sum.z, sum.w};
                if constexpr (EPI == static_cast<int>(Epi::kStoreBF16)) {
                    uint16_t *out = static_cast<uint16_t *>(g.D) + c * g.ldd + r;
                    const f32x2 lo = {sum.x, sum.y}, hi = {sum.z, sum.w};
                    const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
                    const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
                    if (r + 4 <= g.R) {
                        store8(out, make_uint2(w0, w1), g.stream_out);
                    } else {
                        const uint32_t ww[2] = {w0, w1};
                        for (int e = 0; e < 4 && r + e < g.R; ++e)
                            out[e] = static_cast<uint16_t>(ww[e >> 1] >> (16 * (e & 1)));
                    }
                } else {
                    float *out = static_cast<float *>(g.D) + c * g.ldd + r;
                    if (r + 4 <= g.R) {
                        store16(out, sum, g.stream_out);
                    } else {
                        for (int e = 0; e < 4 && r + e < g.R; ++e)
                            out[e] = vv[e];
                    }
                }
            }
            // red is rewritten only after the next group's last stage, past
            // at least one more barrier.
        }
    }
}

// gemm_rows applies: at most 16 tokens, K a multiple of 512, and 32-bit
// buffer offsets for 32 W rows and 16 x rows plus K.  It is routed where it
// measured ahead of gemm_small on MI355X (same box, V = 32768): K >= 8192
// (+9 to +19 %, W larger than the 256 MB MALL).  At K <= 4096 it was 8 - 14 %
// behind (W stays in the MALL between calls) and, with 32 staged tokens,
// 3 % behind at M = 32, so gemm_small keeps those shapes.
bool rows_fits(const GemmProblem &p)
{
    return p.C >= 1 && p.C <= 16 && p.P >= 512 && p.P % 512 == 0 && p.R >= 1 &&
           (32 * std::max(p.lda, p.ldb) + p.P) * 2 < (int64_t(1) << 31);
}

bool rows_preferred(const GemmProblem &p)
{
    return rows_fits(p) && p.P >= 8192;
}

hipError_t launch_rows(const GemmProblem &p, Epi epi, hipStream_t s)
{
    const int64_t ngroups = (p.R + 31) / 32;
    const int64_t target_wg = 256;
    const int gpw = static_cast<int>(std::max<int64_t>(1, (ngroups + target_wg - 1) / target_wg));
    const unsigned nwg = static_cast<unsigned>((ngroups + gpw - 1) / gpw);
    if (epi == Epi::kStoreBF16)
        hipLaunchKernelGGL((gemm_rows<1>), dim3(nwg), dim3(256), 0, s, p, gpw);
    else
        hipLaunchKernelGGL((gemm_rows<0>), dim3(nwg), dim3(256), 0, s, p, gpw);
    return hipGetLastError();
}

hipError_t launch_pp(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    TileMap tm;
    tm.tiles_r = static_cast<int>((p.R + 255) / 256);
    tm.tiles_c = static_cast<int>((p.C + 255) / 256);
    tm.group_r = std::min(std::max(group_r, 1), std::max(tm.tiles_r, 1));
    const int64_t nwg = static_cast<int64_t>(tm.tiles_r) * tm.tiles_c;
    if (nwg == 0)
        return hipSuccess;
    const dim3 grid(static_cast<unsigned>(nwg)), block(512);
    if (epi == Epi::kStoreBF16)
        hipLaunchKernelGGL((gemm_pp<1>), grid, block, 0, s, p, tm);
    else if (epi == Epi::kStoreF32Stats)
        hipLaunchKernelGGL((gemm_pp<3>), grid, block, 0, s, p, tm);
    else
        hipLaunchKernelGGL((gemm_pp<0>), grid, block, 0, s, p, tm);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gemm_wg2: wgrad for few tokens, two workgroups per CU.  With M <= 256 the
// weight gradient is bound by its FP32 dW stores: a 256 x 256 tile computes
// for a few microseconds and then stores 256 KiB, and with gemm_big's 128 KiB
// of LDS a CU holds one workgroup, so its stores and the next tile's loads and
// MFMAs take turns.  Here a tile is 256 (K) x 128 (V), four waves of 128 x 64
// (128 accumulators per lane), and the contraction over tokens runs through a
// single 64-deep LDS stage (A [64][256] + B [64][128], 48 KiB) inside a 64 KiB
// area that the epilogue reuses for its two staging buffers; two workgroups
// fit on a CU, so one's stores overlap the other's loads and MFMAs.  Both
// operands are p-major (x [M][K], dlogits [M][V]) and go through the
// transposing LDS reads of TrOperand; edge tiles and a ragged last stage use
// its guarded register path.
template <int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_wg2(GemmProblem g, TileMap tm)
{
    constexpr int BR = 256, BC = 128, BK = 64, WR = 2, WC = 2, NW = 4, NT = 256;
    constexpr int TR = BR / WR, TC = BC / WC, FR = TR / 32, FC = TC / 32;
    using OpA = TrOperand<BR, BK, NW>;
    using OpB = TrOperand<BC, BK, NW>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 32 * BR * 2];  // 64 KiB
    uint16_t *const sA = lds;                  // [BK][BR]
    uint16_t *const sB = lds + BK * BR;        // [BK][BC]
    static_assert(BK * BR + BK * BC <= 2 * 32 * BR * 2, "stage inside the staging area");

    int tr, tc;
    map_tile(tm, tr, tc);
    const int64_t r0 = static_cast<int64_t>(tr) * BR;
    const int64_t c0 = static_cast<int64_t>(tc) * BC;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WR;
    const int wc = wave / WR;
    const bool interior = r0 + BR <= g.R && c0 + BC <= g.C;

    OpA opA;
    OpB opB;
    opA.init(g.A, g.lda, r0, g.R, g.P, wave, lane, wr * TR);
    opB.init(g.B, g.ldb, c0, g.C, g.P, wave, lane, wc * TC);

    f32x16 acc[FR][FC];
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FC; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    const int64_t nk = (g.P + BK - 1) / BK;
    const int64_t nfull = g.P / BK;
    for (int64_t kt = 0; kt < nk; ++kt) {
        if (interior && kt < nfull) {
            opA.dma(sA, kt * BK, wave);
            opB.dma(sB, kt * BK, wave);
        } else {
            opA.template staged<NT>(sA, kt * BK, tid);
            opB.template staged<NT>(sB, kt * BK, tid);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 fa[FR], fb[FC];
#pragma unroll
            for (int i = 0; i < FR; ++i)
                fa[i] = opA.frag(sA, i, kk);
#pragma unroll
            for (int j = 0; j < FC; ++j)
                fb[j] = opB.frag(sB, j, kk);
#pragma unroll
            for (int i = 0; i < FR; ++i)
#pragma unroll
                for (int j = 0; j < FC; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                        0, 0, 0);
        }
        // Every wave's reads of this stage are done before the next overwrite.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    store_tile_lds<FR, FC, WR, WC, BR, BC, EPI>(g, acc, r0, c0, wr, wc, lane, wave, lds,
                                                lds + 32 * BR * 2);
}

hipError_t launch_wg2(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    TileMap tm;
    tm.tiles_r = static_cast<int>((p.R + 255) / 256);
    tm.tiles_c = static_cast<int>((p.C + 127) / 128);
    tm.group_r = std::min(std::max(group_r, 1), std::max(tm.tiles_r, 1));
    const int64_t nwg = static_cast<int64_t>(tm.tiles_r) * tm.tiles_c;
    if (nwg == 0)
        return hipSuccess;
    const dim3 grid(static_cast<unsigned>(nwg)), block(256);
    if (epi == Epi::kAccumF32)
        hipLaunchKernelGGL((gemm_wg2<2>), grid, block, 0, s, p, tm);
    else if (epi == Epi::kStoreF32)
        hipLaunchKernelGGL((gemm_wg2<0>), grid, block, 0, s, p, tm);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gemm_persist: persistent GEMM over whole 256 x 256 tiles (R and C multiples
// of 256, P a multiple of 128) with a store epilogue -- wgrad (TRANS: both
// operands p-major) and the logits GEMM (both contraction-contiguous).  Each
// tile's output (256 KiB of FP32) takes several microseconds to drain; here
// it overlaps the next tile's work:
//  * one 8-wave workgroup per CU (128 KiB of stage buffers + a 32 KiB
//    epilogue area) walks its XCD's share of the tiles in order, so the
//    next tile's first two 64-deep stages are loaded while the finished tile
//    is written out;
//  * each wave writes its 64 x 128 block through a private 4 KiB LDS area,
//    one 32 x 32 fragment at a time (row-major writes, then whole 128-byte
//    FP32 or 64-byte BF16 row pieces per store instruction), with no
//    workgroup barrier, so the stores stay in flight into the next tile;
//  * only the four waves of wave column 0 issue the direct loads (16 per
//    stage each) and wait on them: vmcnt retires a wave's loads and stores in
//    issue order, so a wait on a stage also waits on that wave's earlier
//    stores, and the other four waves' stores never hold up a stage.
// Stage s of a tile sits in LDS buffer s % 2 (the stage count is even, so
// every tile starts in buffer 0).  Loads are issued from inline assembly,
// untracked by the compiler; the waits count them exactly.  In its 32 x 32 x
// 16 form (wgrad, and the logits GEMM below 1024 tokens) the operand layouts,
// MFMA order and accumulation order are gemm_big's 256 x 256 tile's, so the
// two give bitwise-identical output; the logits GEMM from 1024 tokens on runs
// the 16 x 16 x 32 form (MF16), which sums each output in another order.
__device__ __forceinline__ int persist_swz(int row)
{
    // 16-byte chunk key of a 128-byte row: distinct over any 8 consecutive
    // rows, and (chunk, row parity) distinct over any 16.
    return (row & 7) ^ ((row >> 3) & 1);
}

template <bool TRANS, int EPI, bool MF16>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_persist(GemmProblem g, TileMap tm, int per_xcd)
{
    constexpr int BR = 256, BC = 256, BK = 64, WR = 4, NL = 4;
    constexpr int TR = 64, TC = 128, FR = TR / 32, FC = TC / 32;
    constexpr bool BF = EPI == static_cast<int>(Epi::kStoreBF16);
    static_assert(EPI == static_cast<int>(Epi::kStoreF32) || BF, "store epilogues only");
    // p-major operands (wgrad: x [M][K], dlogits [M][V]) are read through
    // transposing LDS loads; contraction-contiguous ones (logits: W [V][K],
    // x [M][K]) keep gemm_big's k-contiguous stage layout.
    using OpA = std::conditional_t<TRANS, TrOperand<BR, BK, NL>, DmaOperand<BR, BK, NL>>;
    using OpB = std::conditional_t<TRANS, TrOperand<BC, BK, NL>, DmaOperand<BC, BK, NL>>;
    constexpr int NDMA = OpA::NB + OpB::NB;    // direct loads per loading wave per stage
    constexpr int NST = FR * FC * (BF ? 2 : 4);  // stores per wave per tile
    // MF16: the 16 x 16 x 32 MFMA form (contraction-contiguous operands only);
    // its epilogue issues the same NST stores per wave per tile.
    static_assert(!(MF16 && TRANS), "the 16 x 16 form reads k-contiguous stages");
    __shared__ __attribute__((aligned(16))) uint16_t sA0[BR * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sA1[BR * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB0[BC * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB1[BC * BK];
    __shared__ __attribute__((aligned(16))) float sE[8 * 32 * 32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WR;
    const int wc = wave / WR;
    const bool loads = wc == 0;
    // Workgroups b, b + 8, ... share an XCD; XCD x takes the tiles
    // [x per_xcd, (x + 1) per_xcd) of the grouped order, gridDim.x / 8 at a
    // time.
    const int xcd = blockIdx.x % kXcds;
    const int slots = gridDim.x / kXcds;
    auto decode = [&](int j, int64_t &r0, int64_t &c0) {
        const int v = xcd * per_xcd + j;
        const int gsz = tm.group_r * tm.tiles_c;
        const int gi = v / gsz;
        const int first_r = gi * tm.group_r;
        const int rows_in_group = min(tm.tiles_r - first_r, tm.group_r);
        const int in = v - gi * gsz;
        r0 = static_cast<int64_t>(first_r + in % rows_in_group) * BR;
        c0 = static_cast<int64_t>(in / rows_in_group) * BC;
    };

    // Per-lane direct-load offsets, the same for every tile (all tiles are
    // whole): computed for the tile at row 0.
    OpA opA;
    OpB opB;
    if constexpr (TRANS) {
        opA.init(g.A, g.lda, 0, g.R, g.P, wr, lane, wr * TR);
        opB.init(g.B, g.ldb, 0, g.C, g.P, wr, lane, wc * TC);
    } else {
        opA.init(g.A, g.lda, 0, g.R, g.P, wr, lane);
        opB.init(g.B, g.ldb, 0, g.C, g.P, wr, lane);
    }
    // Stage kt of the tile at (r0, c0) into (lA, lB), by the loading waves.
    auto dma = [&](uint16_t *lA, uint16_t *lB, int64_t r0, int64_t c0, int64_t kt) {
        if (!loads)
            return;
        __amdgpu_buffer_rsrc_t ra, rb;
        int soff;
        if constexpr (TRANS) {
            ra = tile_rsrc(g.A + kt * BK * g.lda + r0);
            rb = tile_rsrc(g.B + kt * BK * g.ldb + c0);
            soff = 0;
        } else {
            ra = tile_rsrc(g.A + r0 * g.lda);
            rb = tile_rsrc(g.B + c0 * g.ldb);
            soff = static_cast<int>(kt * BK * 2);
        }
#pragma unroll
        for (int i = 0; i < OpA::NB; ++i)
            dma16_untracked(ra, lds_addr(lA + (wr * OpA::NB + i) * 512), opA.off[i], soff);
#pragma unroll
        for (int i = 0; i < OpB::NB; ++i)
            dma16_untracked(rb, lds_addr(lB + (wr * OpB::NB + i) * 512), opB.off[i], soff);
    };

    // k-contiguous layout: fragment i of the wave covers tile rows
    // wr*TR + 32i + lane%32; its chunk key depends on i only through parity.
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const int fbA = (wr * TR + lrow) * BK;
    const int fbB = (wc * TC + lrow) * BK;
    int keyA[2], keyB[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        keyA[par] = khalf ^ lds_swz<BK>(wr * TR + par * 32 + lrow);
        keyB[par] = khalf ^ lds_swz<BK>(wc * TC + par * 32 + lrow);
    }
    bf16x8 fa[2][FR], fb[2][FC];
    auto frag_load = [&](const uint16_t *lA, const uint16_t *lB, int kk, int sl) {
#pragma unroll
        for (int i = 0; i < FR; ++i) {
            if constexpr (TRANS)
                fa[sl][i] = opA.frag(lA, i, kk);
            else
                fa[sl][i] = *reinterpret_cast<const bf16x8 *>(
                    &lA[fbA + i * 32 * BK + (((2 * kk) ^ keyA[i & 1]) * 8)]);
        }
#pragma unroll
        for (int j = 0; j < FC; ++j) {
            if constexpr (TRANS)
                fb[sl][j] = opB.frag(lB, j, kk);
            else
                fb[sl][j] = *reinterpret_cast<const bf16x8 *>(
                    &lB[fbB + j * 32 * BK + (((2 * kk) ^ keyB[j & 1]) * 8)]);
        }
    };
    f32x16 acc[FR][FC];
    auto mfma_rows = [&](int sl, int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < FC; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][i], fb[sl][j],
                                                                    acc[i][j], 0, 0, 0);
    };
    // The MFMAs of one stage whose k-step-0 fragments are in slot 0, fragment
    // reads one k step ahead; the last half row of MFMAs is left to the
    // caller, to run behind its wait and barrier.
    auto stage_mfma = [&](const uint16_t *cA, const uint16_t *cB) {
        frag_load(cA, cB, 1, 1);
        mfma_rows(0, 0, FR);
        frag_load(cA, cB, 2, 0);
        mfma_rows(1, 0, FR);
        frag_load(cA, cB, 3, 1);
        mfma_rows(0, 0, FR);
        mfma_rows(1, 0, FR / 2);
    };
    // Hand-off between stages: the loading waves wait until at most N of
    // their memory operations are in flight, then every wave's LDS reads are
    // done and the workgroup meets.
    auto hand_off = [&](auto nc) {
        __builtin_amdgcn_sched_barrier(0);
        if (loads)
            vm_wait<decltype(nc)::value>();
        pp_barrier();
    };

    const int cl = lane & 31, hl = lane >> 5;
    float *const own = sE + wave * 32 * 32;
    auto epilogue = [&](int64_t r0, int64_t c0) {
#pragma unroll
        for (int t = 0; t < FC; ++t)
#pragma unroll
            for (int i = 0; i < FR; ++i) {
                // Lane (cl, hl) holds rows 8q + 4hl .. + 3 of output row cl.
                if constexpr (BF) {
                    // 32 rows of 64 bytes; 16-byte chunk q of row c at q ^ ((c >> 2) & 3).
                    char *ob = reinterpret_cast<char *>(own);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x2 lo = {acc[i][t][4 * q + 0], acc[i][t][4 * q + 1]};
                        const f32x2 hi = {acc[i][t][4 * q + 2], acc[i][t][4 * q + 3]};
                        uint2 w;
                        w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
                        w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
                        *reinterpret_cast<uint2 *>(ob + cl * 64 + ((q ^ ((cl >> 2) & 3)) << 4) +
                                                   hl * 8) = w;
                    }
                    // Four lanes per 64-byte row, sixteen rows per store.
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int rr = 16 * s + (lane >> 2), kc = lane & 3;
                        const uint4 v = *reinterpret_cast<const uint4 *>(
                            ob + rr * 64 + ((kc ^ ((rr >> 2) & 3)) << 4));
                        uint16_t *out = static_cast<uint16_t *>(g.D) +
                                        (c0 + wc * TC + t * 32 + rr) * g.ldd + r0 + wr * TR +
                                        i * 32 + 8 * kc;
                        store16(out, v, true);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float4 v;
                        v.x = acc[i][t][4 * q + 0];
                        v.y = acc[i][t][4 * q + 1];
                        v.z = acc[i][t][4 * q + 2];
                        v.w = acc[i][t][4 * q + 3];
                        *reinterpret_cast<float4 *>(
                            &own[cl * 32 + (((2 * q + hl) ^ persist_swz(cl)) << 2)]) = v;
                    }
                    // Eight lanes per 128-byte row, eight rows per store.
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int rr = 8 * s + (lane >> 3), kc = lane & 7;
                        const float4 v = *reinterpret_cast<const float4 *>(
                            &own[rr * 32 + ((kc ^ persist_swz(rr)) << 2)]);
                        float *out = static_cast<float *>(g.D) +
                                     (c0 + wc * TC + t * 32 + rr) * g.ldd + r0 + wr * TR +
                                     i * 32 + 4 * kc;
                        store16(out, v, true);
                    }
                }
            }
    };

    if constexpr (MF16) {
        // 16 x 16 x 32 form.  Fragment i of A covers wave rows 16 i .. 16 i + 15
        // (lane l: row l % 16, the 8 contraction values from 8 (l / 16) of the
        // 32-wide k step), fragment jj of B the tokens 16 jj .. 16 jj + 15; lane l
        // then holds outputs (rows 16 i + 4 (l / 16) .. + 3, token 16 jj + l % 16).
        // A 64-deep stage is two k steps of 4 x 8 MFMAs.  Each fragment
        // register is reloaded for the next k step as soon as its last MFMA of
        // the current one is issued (A: after its row, B: after the last row),
        // so one set of fragment registers suffices; the next stage's first
        // fragments are read behind the hand-off, which sits after the first
        // three rows of k step 1 (after two it measured 1 - 5 % slower).
        // Against the 32 x 32 x 16 form the matrix pipe moves half the
        // accumulator bytes per FLOP, which at the board's power cap buys clock.
        constexpr int GR = TR / 16, GC = TC / 16;
        const int q16 = lane >> 4, t16 = lane & 15;
        const int rA = wr * TR + t16, rB = wc * TC + t16;
        // Stage rows here take the key r % 8 (chunk c of row r at c ^ (r % 8)),
        // not lds_swz: a fragment read of this form (16 rows x 4 chunks) is
        // free of bank conflicts with it and conflicts with lds_swz's XOR key
        // (measured: 50 M conflict cycles per launch at M=1024 K=8192).  The
        // key of every fragment row is t16 % 8, so one per-lane term serves all.
        const int v16 = q16 ^ (t16 & 7);
        bf16x8 ga[GR], gb[GC];
        f32x4 acc4[GR][GC];
        auto ldA = [&](const uint16_t *l, int i, int h) {
            ga[i] = *reinterpret_cast<const bf16x8 *>(&l[(rA + 16 * i) * BK + ((v16 ^ (4 * h)) << 3)]);
        };
        auto ldB = [&](const uint16_t *l, int jj, int h) {
            gb[jj] = *reinterpret_cast<const bf16x8 *>(&l[(rB + 16 * jj) * BK + ((v16 ^ (4 * h)) << 3)]);
        };
        auto mf = [&](int i, int jj) {
            acc4[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[i], gb[jj], acc4[i][jj], 0, 0, 0);
        };
        // k step 0 of the stage in (cA, cB), reloading for its k step 1.
        auto step0 = [&](const uint16_t *cA, const uint16_t *cB) {
#pragma unroll
            for (int i = 0; i < GR; ++i) {
#pragma unroll
                for (int jj = 0; jj < GC; ++jj) {
                    mf(i, jj);
                    if (i == GR - 1)
                        ldB(cB, jj, 1);
                }
                ldA(cA, i, 1);
            }
        };
        constexpr int HEAD = GR - 1;  // rows of k step 1 before the hand-off
        auto step1_head = [&]() {
#pragma unroll
            for (int i = 0; i < HEAD; ++i)
#pragma unroll
                for (int jj = 0; jj < GC; ++jj)
                    mf(i, jj);
        };
        // The rest of k step 1, loading k step 0 of the next stage (nA, nB)
        // when NEXT (the last stage of a tile has none).
        auto step1_tail = [&](auto nextc, const uint16_t *nA, const uint16_t *nB) {
            constexpr bool NEXT = decltype(nextc)::value;
            if constexpr (NEXT) {
#pragma unroll
                for (int i = 0; i < HEAD; ++i)
                    ldA(nA, i, 0);
            }
#pragma unroll
            for (int i = HEAD; i < GR; ++i) {
#pragma unroll
                for (int jj = 0; jj < GC; ++jj) {
                    mf(i, jj);
                    if constexpr (NEXT)
                        if (i == GR - 1)
                            ldB(nB, jj, 0);
                }
                if constexpr (NEXT)
                    ldA(nA, i, 0);
            }
        };
        // Each wave writes its 64 x 128 block through its 4 KiB LDS area, 16
        // tokens at a time: FP32 rows of 256 bytes (16-byte chunk k of row t at
        // k ^ t, four rows per store instruction), BF16 rows of 128 bytes
        // (chunk k at k ^ (t % 8), eight rows per store): NST stores per tile.
        char *const ownb = reinterpret_cast<char *>(sE + wave * 32 * 32);
        auto epilogue16 = [&](int64_t r0, int64_t c0) {
#pragma unroll
            for (int jj = 0; jj < GC; ++jj) {
                if constexpr (BF) {
#pragma unroll
                    for (int i = 0; i < GR; ++i) {
                        const f32x2 lo = {acc4[i][jj][0], acc4[i][jj][1]};
                        const f32x2 hi = {acc4[i][jj][2], acc4[i][jj][3]};
                        uint2 w;
                        w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
                        w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
                        *reinterpret_cast<uint2 *>(ownb + t16 * 128 +
                                                   (((2 * i + (q16 >> 1)) ^ (t16 & 7)) << 4) +
                                                   (q16 & 1) * 8) = w;
                    }
#pragma unroll
                    for (int sx = 0; sx < 2; ++sx) {
                        const int rr = 8 * sx + (lane >> 3), kc = lane & 7;
                        const uint4 v = *reinterpret_cast<const uint4 *>(
                            ownb + rr * 128 + ((kc ^ (rr & 7)) << 4));
                        uint16_t *out = static_cast<uint16_t *>(g.D) +
                                        (c0 + wc * TC + 16 * jj + rr) * g.ldd + r0 + wr * TR + 8 * kc;
                        store16(out, v, true);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < GR; ++i) {
                        float4 v;
                        v.x = acc4[i][jj][0];
                        v.y = acc4[i][jj][1];
                        v.z = acc4[i][jj][2];
                        v.w = acc4[i][jj][3];
                        *reinterpret_cast<float4 *>(ownb + t16 * 256 + (((4 * i + q16) ^ t16) << 4)) = v;
                    }
#pragma unroll
                    for (int sx = 0; sx < 4; ++sx) {
                        const int rr = 4 * sx + q16, kc = t16;
                        const float4 v = *reinterpret_cast<const float4 *>(
                            ownb + rr * 256 + ((kc ^ rr) << 4));
                        float *out = static_cast<float *>(g.D) +
                                     (c0 + wc * TC + 16 * jj + rr) * g.ldd + r0 + wr * TR + 4 * kc;
                        store16(out, v, true);
                    }
                }
            }
        };
        static_assert(GC * (BF ? 2 : 4) == NST, "the 16 x 16 epilogue issues NST stores");
        // Direct loads as DmaOperand's, with the key above and the offsets
        // recomputed per load rather than held in registers: block b (8 rows)
        // of a stage, lane l at row 8 b + l / 8, chunk (l % 8) ^ (l / 8).
        const int dl_row = lane >> 3, dl_key = (lane & 7) ^ dl_row;
        auto dma16 = [&](uint16_t *lA, uint16_t *lB, int64_t r0, int64_t c0, int64_t kt) {
            if (!loads)
                return;
            const __amdgpu_buffer_rsrc_t ra = tile_rsrc(g.A + r0 * g.lda);
            const __amdgpu_buffer_rsrc_t rb = tile_rsrc(g.B + c0 * g.ldb);
            const int soff = static_cast<int>(kt * BK * 2);
#pragma unroll
            for (int i = 0; i < OpA::NB; ++i) {
                const int b = wr * OpA::NB + i;
                const uint32_t voff =
                    static_cast<uint32_t>(((b * 8 + dl_row) * g.lda + (dl_key << 3)) * 2);
                dma16_untracked(ra, lds_addr(lA + b * 512), voff, soff);
            }
#pragma unroll
            for (int i = 0; i < OpB::NB; ++i) {
                const int b = wr * OpB::NB + i;
                const uint32_t voff =
                    static_cast<uint32_t>(((b * 8 + dl_row) * g.ldb + (dl_key << 3)) * 2);
                dma16_untracked(rb, lds_addr(lB + b * 512), voff, soff);
            }
        };

        const int64_t nk = g.P / BK;  // even, >= 2
        int j = blockIdx.x / kXcds;
        if (j >= per_xcd)
            return;
        int64_t r0, c0;
        decode(j, r0, c0);
        dma16(sA0, sB0, r0, c0, 0);
        dma16(sA1, sB1, r0, c0, 1);
        bool first = true;
        const std::true_type with_next;
        const std::false_type no_next;
        for (;;) {
            const std::integral_constant<int, NDMA> after_s0_first;
            const std::integral_constant<int, NDMA + NST> after_s0;
            if (first)
                hand_off(after_s0_first);
            else
                hand_off(after_s0);
#pragma unroll
            for (int i = 0; i < GR; ++i)
#pragma unroll
                for (int jj = 0; jj < GC; ++jj)
                    acc4[i][jj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < GR; ++i)
                ldA(sA0, i, 0);
#pragma unroll
            for (int jj = 0; jj < GC; ++jj)
                ldB(sB0, jj, 0);
            const int jn = j + slots;
            const bool has_next = jn < per_xcd;
            int64_t nr0 = 0, nc0 = 0;
            if (has_next)
                decode(jn, nr0, nc0);
            step0(sA0, sB0);
            step1_head();
            const std::integral_constant<int, 0> none;
            const std::integral_constant<int, NST> after_s1;
            if (first)
                hand_off(none);
            else
                hand_off(after_s1);
            step1_tail(with_next, sA1, sB1);
            int64_t kt = 1;
            for (; kt + 2 < nk; kt += 2) {
                dma16(sA0, sB0, r0, c0, kt + 1);
                step0(sA1, sB1);
                step1_head();
                hand_off(none);
                step1_tail(with_next, sA0, sB0);
                dma16(sA1, sB1, r0, c0, kt + 2);
                step0(sA0, sB0);
                step1_head();
                hand_off(none);
                step1_tail(with_next, sA1, sB1);
            }
            if (has_next)
                dma16(sA0, sB0, nr0, nc0, 0);
            step0(sA1, sB1);
            step1_head();
            step1_tail(no_next, nullptr, nullptr);
            pp_barrier();
            if (has_next)
                dma16(sA1, sB1, nr0, nc0, 1);
            epilogue16(r0, c0);
            if (!has_next)
                break;
            j = jn, r0 = nr0, c0 = nc0;
            first = false;
        }
        return;
    }
    const int64_t nk = g.P / BK;  // even, >= 2
    int j = blockIdx.x / kXcds;
    if (j >= per_xcd)
        return;
    int64_t r0, c0;
    decode(j, r0, c0);
    // In flight at the top of a tile, in issue order: stage 0 (NDMA), stage 1
    // (NDMA) and, after the first tile, the previous tile's NST stores.
    dma(sA0, sB0, r0, c0, 0);
    dma(sA1, sB1, r0, c0, 1);
    bool first = true;
    for (;;) {
        const std::integral_constant<int, NDMA> after_s0_first;
        const std::integral_constant<int, NDMA + NST> after_s0;
        if (first)
            hand_off(after_s0_first);
        else
            hand_off(after_s0);
#pragma unroll
        for (int i = 0; i < FR; ++i)
#pragma unroll
            for (int jx = 0; jx < FC; ++jx)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[i][jx][e] = 0.0f;
        frag_load(sA0, sB0, 0, 0);
        const int jn = j + slots;
        const bool has_next = jn < per_xcd;
        int64_t nr0 = 0, nc0 = 0;
        if (has_next)
            decode(jn, nr0, nc0);
        // Stage 0 (buffer 0); stage 1 is already on its way into buffer 1.
        stage_mfma(sA0, sB0);
        const std::integral_constant<int, 0> none;
        const std::integral_constant<int, NST> after_s1;
        if (first)
            hand_off(none);
        else
            hand_off(after_s1);
        frag_load(sA1, sB1, 0, 0);
        mfma_rows(1, FR / 2, FR);
        // Stages 1 .. nk - 2 in pairs: each loads the stage after it into the
        // buffer the previous stage freed.
        int64_t kt = 1;
        for (; kt + 2 < nk; kt += 2) {
            dma(sA0, sB0, r0, c0, kt + 1);
            stage_mfma(sA1, sB1);
            hand_off(none);
            frag_load(sA0, sB0, 0, 0);
            mfma_rows(1, FR / 2, FR);
            dma(sA1, sB1, r0, c0, kt + 2);
            stage_mfma(sA0, sB0);
            hand_off(none);
            frag_load(sA1, sB1, 0, 0);
            mfma_rows(1, FR / 2, FR);
        }
        // Last stage (buffer 1): the next tile's stage 0 goes into buffer 0
        // now, its stage 1 into buffer 1 once every wave has read it.
        if (has_next)
            dma(sA0, sB0, nr0, nc0, 0);
        stage_mfma(sA1, sB1);
        mfma_rows(1, FR / 2, FR);
        pp_barrier();
        if (has_next)
            dma(sA1, sB1, nr0, nc0, 1);
        epilogue(r0, c0);
        if (!has_next)
            break;
        j = jn, r0 = nr0, c0 = nc0;
        first = false;
    }
}

// gemm_persist's shapes: whole tiles, an even number of 64-deep stages, and
// at least two tiles per CU in whole groups of eight (one range per XCD).
bool persist_fits(const GemmProblem &p)
{
    if (p.psplit != 0 || p.R % 256 != 0 || p.C % 256 != 0 || p.P % 128 != 0 || p.P == 0)
        return false;
    const int64_t tiles = (p.R / 256) * (p.C / 256);
    return tiles >= 512 && tiles % kXcds == 0;
}

template <bool TRANS>
hipError_t launch_persist(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    TileMap tm;
    tm.tiles_r = static_cast<int>(p.R / 256);
    tm.tiles_c = static_cast<int>(p.C / 256);
    tm.group_r = std::min(std::max(group_r, 1), tm.tiles_r);
    const int per_xcd = tm.tiles_r * tm.tiles_c / kXcds;
    // The logits GEMM takes the 16 x 16 x 32 form from 1024 tokens on.
    // Measured on MI355X against the 32 x 32 x 16 form (same box; alternated
    // calls / 2 s back to back at the 1400 W cap): M=1024 K=8192 V=32768
    // 445 -> 419 us / 1234 -> 1330 TFLOPS, M=4096 K=8192 1732 -> 1661 us,
    // M=1024 K=16384 870 -> 855 us; but M=512 K=16384 V=131072 1883 -> 2163 us
    // (1180 -> 986 TFLOPS at a higher clock) and M=512 K=8192 V=65536 +5 %.
#ifndef LMH_MF16_MIN_TOKENS
#define LMH_MF16_MIN_TOKENS 1024
#endif
    const bool mf16 = !TRANS && p.C >= LMH_MF16_MIN_TOKENS;
    // One workgroup per CU (160 KiB of LDS each).
    if (epi == Epi::kStoreF32) {
        if constexpr (!TRANS) {
            if (mf16) {
                hipLaunchKernelGGL((gemm_persist<TRANS, 0, true>), dim3(256), dim3(512), 0, s, p, tm, per_xcd);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((gemm_persist<TRANS, 0, false>), dim3(256), dim3(512), 0, s, p, tm, per_xcd);
    } else if (epi == Epi::kStoreBF16) {
        if constexpr (!TRANS) {
            if (mf16) {
                hipLaunchKernelGGL((gemm_persist<TRANS, 1, true>), dim3(256), dim3(512), 0, s, p, tm, per_xcd);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((gemm_persist<TRANS, 1, false>), dim3(256), dim3(512), 0, s, p, tm, per_xcd);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int BR, int BC, int WR, int WC, bool AT, bool BT>
hipError_t launch_big(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    constexpr int BK = 64;
    TileMap tm;
    tm.tiles_r = static_cast<int>((p.R + BR - 1) / BR);
    tm.tiles_c = static_cast<int>((p.C + BC - 1) / BC);
    tm.group_r = std::min(std::max(group_r, 1), std::max(tm.tiles_r, 1));
    const int64_t nwg = static_cast<int64_t>(tm.tiles_r) * tm.tiles_c;
    if (nwg == 0)
        return hipSuccess;
    const unsigned nsplit =
        p.psplit > 0 ? static_cast<unsigned>((p.P + p.psplit - 1) / p.psplit) : 1u;
    dim3 grid(static_cast<unsigned>(nwg), nsplit), block(WR * WC * 64);
    switch (epi) {
    case Epi::kStoreF32:
        hipLaunchKernelGGL((gemm_big<BR, BC, BK, WR, WC, AT, BT, 0>), grid, block, 0, s, p, tm);
        break;
    case Epi::kStoreBF16:
        hipLaunchKernelGGL((gemm_big<BR, BC, BK, WR, WC, AT, BT, 1>), grid, block, 0, s, p, tm);
        break;
    case Epi::kAccumF32:
        hipLaunchKernelGGL((gemm_big<BR, BC, BK, WR, WC, AT, BT, 2>), grid, block, 0, s, p, tm);
        break;
    case Epi::kStoreF32Stats:
        if constexpr (!AT && !BT && BR == 256 && WR == 4)
            hipLaunchKernelGGL((gemm_big<BR, BC, BK, WR, WC, AT, BT, 3>), grid, block, 0, s, p, tm);
        else
            return hipErrorInvalidValue;
        break;
    }
    return hipGetLastError();
}

template <int BR, int BC, int WR, int WC, bool AT, bool BT>
hipError_t launch_cfg(const GemmProblem &p, Epi epi, int group_r, hipStream_t s)
{
    constexpr int BK = 64;
    TileMap tm;
    tm.tiles_r = static_cast<int>((p.R + BR - 1) / BR);
    tm.tiles_c = static_cast<int>((p.C + BC - 1) / BC);
    tm.group_r = std::min(std::max(group_r, 1), std::max(tm.tiles_r, 1));
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
    case Epi::kStoreF32Stats:  // never routed here (see launch_gemm_logits)
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// The large-tile kernel addresses a tile through 32-bit byte offsets: its
// span must stay below 2^31 bytes (256 rows of the operand plus one stage).
static bool big_offsets_fit(const GemmProblem &p)
{
    return (256 * std::max(p.lda, p.ldb) + 64) * 2 < (int64_t(1) << 31) &&
           (64 * std::max(p.lda, p.ldb) + 256) * 2 < (int64_t(1) << 31);
}

#ifndef LMH_SMALLM_CFG
#define LMH_SMALLM_CFG 0
#endif

// The many-token logits kernels (gemm_pp, gemm_big 256 x 256 with 8 waves)
// also write the cross-entropy records in their epilogue.
bool gemm_logits_stats_in_epilogue(const GemmProblem &p)
{
    return big_offsets_fit(p) && LMH_SMALLM_CFG == 0 && p.C > 256;
}

hipError_t launch_gemm_logits(const GemmProblem &p, Epi epi, hipStream_t s)
{
    // R = V (vocabulary), C = M (tokens); both operands K-contiguous.
    if (epi == Epi::kStoreF32Stats && !gemm_logits_stats_in_epilogue(p))
        epi = Epi::kStoreF32;  // the caller derives the records from the logits
    if (!big_offsets_fit(p))
        return launch_cfg<128, 128, 2, 2, false, false>(p, epi, 8, s);
    switch (LMH_SMALLM_CFG) {  // pinned shapes for tuning builds
    case 1: return launch_big<128, 128, 2, 2, false, false>(p, epi, 8, s);
    case 2: return launch_small<128, 4>(p, epi, 8, s);
    case 3: return launch_small<64, 6>(p, epi, 8, s);
    case 4: return launch_small<32, 6>(p, epi, 8, s);
    case 5: return launch_big<256, 256, 4, 2, false, false>(p, epi, 8, s);
    default: break;
    }
#ifndef LMH_SMALL_S32
#define LMH_SMALL_S32 8
#endif
#ifndef LMH_SMALL_S128
#define LMH_SMALL_S128 5
#endif
#ifndef LMH_ROWS
#define LMH_ROWS 1
#endif
    if ((LMH_ROWS == 2 ? rows_fits(p) : LMH_ROWS && rows_preferred(p)) &&
        (epi == Epi::kStoreF32 || epi == Epi::kStoreBF16))
        return launch_rows(p, epi, s);
    // Up to 64 tokens with K <= 4096: 128-deep stages, so each W row is read
    // in 256-byte runs (rings of 4 and 3 stages fill the 160 KiB of LDS).
    // Measured on two MI355X against 64-deep stages, V=32768: K=4096 -6 to
    // -10 % (M=16, 32, 64), M=64 K=1024 -11 to -13 %, other K <= 4096 within
    // 1 % (M=32 K=1024 +2.5 % on one of the two); at K=8192 0 to +4 %.
    if (p.C <= 32)
        return p.P <= 4096 ? launch_small<32, 4, 128>(p, epi, 8, s)
                           : launch_small<32, LMH_SMALL_S32>(p, epi, 8, s);
    if (p.C <= 64)
        return p.P <= 4096 ? launch_small<64, 3, 128>(p, epi, 8, s)
                           : launch_small<64, 6>(p, epi, 8, s);
    if (p.C <= 128)
        return launch_small<128, LMH_SMALL_S128>(p, epi, 8, s);
    // 129 - 256 tokens: one 256-token tile column (ring of 3 stages of 48
    // KiB), so each W row block is streamed by one workgroup instead of two.
    // Measured on MI355X against two 128-token columns (V=32768, FP32 out,
    // medians of 40 alternated): M=256 K=1024 36.3 -> 30.4 us, K=4096 94.6
    // -> 85.2, K=8192 204.4 -> 169.9; M=160 and 192 -6 to -17 %.
    if (p.C <= 256)
        return launch_small<256, 3>(p, epi, 8, s);
    // Many tokens: the ping-pong ring kernel for K <= 2048 or at most 384
    // tokens, gemm_big otherwise.  Measured on MI355X (V=32768, medians of 15,
    // three alternated rounds), gemm_pp -> gemm_big: M=1024 K=1024 79.6-80.6
    // -> 82.0-83.1 us, K=2048 126.6-138.7 -> 128.1-143.1, K=4096 240.6-249.5
    // -> 229.6-241.3, K=8192 482.6-490.4 -> 463.7-469.9; M=384 K=8192
    // 230.2-235.0 -> 237.2-242.2; M=512 K=4096 133.5-134.7 -> 129.8-130.2;
    // M=2048 K=4096 460.7-470.6 -> 455.1-461.8; M=4096 K=8192 1878-1882 ->
    // 1825-1839; M=1024 K=8192 V=131072 1899-1932 -> 1850-1865.
#ifndef LMH_PP
#define LMH_PP 1
#endif
    // Whole tiles (V and M multiples of 256, K of 128, at least 512 tiles):
    // the persistent kernel, whose output stores overlap the next tile.
    // Measured on MI355X against the routing below (bitwise-identical output,
    // FP32 out, V=32768, three rounds of 20): M=1024 K=1024 82.6-83.3 ->
    // 78.8-79.7 us, K=2048 131.9-135.4 -> 127.0-128.5, K=4096 239.9-241.9 ->
    // 244.1-246.0, K=8192 479.7-485.0 -> 461.3-467.7, K=16384 929-932 ->
    // 920-923; M=2048 K=4096 468-477 -> 457-462; M=4096 K=8192 1879-1894 ->
    // 1849-1857; M=1024 K=8192 V=131072 1883-1899 -> 1846-1854.
#ifndef LMH_LOGITS_PERSIST
#define LMH_LOGITS_PERSIST 1
#endif
    // Its tile order walks 4 tile rows (V) before stepping along M.  Measured
    // on MI355X against 8 (bitwise-identical output, medians of 15 alternated
    // calls): M=4096 K=8192 1717 -> 1656 us, M=1024 K=1024 72.7 -> 71.0, M=4096
    // K=16384 V=131072 14058 -> 13969, M=1024 K=8192 equal (the same 32 tiles
    // run at once on each XCD); 16 and 32 were 4 - 37 % slower.
    if (LMH_LOGITS_PERSIST && (epi == Epi::kStoreF32 || epi == Epi::kStoreBF16) && persist_fits(p))
        return launch_persist<false>(p, epi, 4, s);
    if (LMH_PP && p.P % 32 == 0 && (p.P <= 2048 || (p.C <= 384 && p.P <= 8192)) &&
        epi != Epi::kAccumF32)
        return launch_pp(p, epi, 8, s);
    return launch_big<256, 256, 4, 2, false, false>(p, epi, 8, s);
}

// dgrad / wgrad tile choice (measured on MI355X at M=1024 K=8192 V=32768 and
// M=4096 K=16384 V=131072): the logits kernel's 256x256 tile with 8 waves
// whenever there are at least 256 such tiles; otherwise (dgrad's short M x K
// output at M=1024) 256x128 tiles with 8 waves, and 128x128 for tiny problems.
template <bool AT, bool BT>
hipError_t launch_bwd(const GemmProblem &p, Epi epi, hipStream_t s)
{
    if (!big_offsets_fit(p))
        return launch_cfg<128, 128, 2, 2, AT, BT>(p, epi, 8, s);
#ifndef LMH_BWD_CFG
#define LMH_BWD_CFG 0
#endif
    switch (LMH_BWD_CFG) {  // pinned tile shapes for tuning builds
    case 1: return launch_big<256, 256, 4, 2, AT, BT>(p, epi, 8, s);
    case 2: return launch_big<256, 256, 2, 2, AT, BT>(p, epi, 8, s);
    case 3: return launch_big<256, 128, 4, 2, AT, BT>(p, epi, 8, s);
    case 4: return launch_big<128, 128, 2, 2, AT, BT>(p, epi, 8, s);
    default: break;
    }
    // wgrad's tile order (tile rows along K walked before stepping along V):
    // with few tokens it is bound by its FP32 dW stores, and walking 16 tile
    // rows -- whole 4096-wide dW row blocks -- writes longer runs of each row.
    // Measured on MI355X against 8: M=128 K=4096 V=32768 -4 %, K=16384 -14 %,
    // M=256 K=16384 -10 %, M=16 K=8192 -7 %; at M=512 K=16384 V=131072 16 was
    // 6 % slower and at M=1024 K=8192 equal, so 8 above 256 tokens.
#ifndef LMH_WGRAD_GROUP
#define LMH_WGRAD_GROUP 0
#endif
    const int wgrad_group = LMH_WGRAD_GROUP > 0 ? LMH_WGRAD_GROUP : (p.P <= 256 ? 16 : 8);
    const int64_t tiles256 = ((p.R + 255) / 256) * ((p.C + 255) / 256);
    const int64_t tiles256x128 = ((p.R + 255) / 256) * ((p.C + 127) / 128);
    // wgrad with at most LMH_WGRAD_WG2 tokens and at least two 256 x 128 tiles
    // per CU: two workgroups per CU (gemm_wg2).  Measured on MI355X against
    // gemm_big's 256 x 256 tiles (bit-identical output): M=16 - 256 -8 to -20 %
    // (M=128 K=4096 V=32768 130.7 -> 116.2 us, K=8192 V=131072 890 -> 711 us),
    // M=384 -6 %, M=512 -2 %, M=768 +0.5 %, M=1024 +3 %, M=2048 +9 %.
#ifndef LMH_WGRAD_WG2
#define LMH_WGRAD_WG2 512
#endif
    if constexpr (AT && BT) {
        // Whole-tile wgrad with the store epilogue: the persistent kernel,
        // whose dW stores overlap the next tile (gemm_persist<true>).  Measured on MI355X against
        // the kernels below (bitwise-identical dW), K=8192 V=32768: M=128
        // 197-215 -> 184-189 us, M=256 259 -> 199-208, M=512 365-369 ->
        // 304-305, M=768 485-488 -> 411-418, M=1024 573-575 -> 514-516,
        // M=4096 1784-1809 -> 1755-1770; K=16384 V=131072: M=128 1477-1594 ->
        // 1427, M=512 2918-3000 -> 2365-2373, M=4096 14217-14241 ->
        // 13687-13760 us.
        if (epi == Epi::kStoreF32 && persist_fits(p))
            return launch_persist<true>(p, epi, wgrad_group, s);
        if (p.P <= LMH_WGRAD_WG2 && tiles256x128 >= 512)
            return launch_wg2(p, epi, wgrad_group, s);
    }
    if (tiles256 >= 256)
        return launch_big<256, 256, 4, 2, AT, BT>(p, epi, BT ? wgrad_group : 8, s);
    if (tiles256x128 >= 192)
        return launch_big<256, 128, 4, 2, AT, BT>(p, epi, 8, s);
    return launch_big<128, 128, 2, 2, AT, BT>(p, epi, 8, s);
}

hipError_t launch_gemm_dgrad(const GemmProblem &p, Epi epi, hipStream_t s)
{
    // R = K (hidden), C = M (tokens), A = W stored [V][K] (p-major).
    return launch_bwd<true, false>(p, epi, s);
}

// dgrad with the sum over V split in `splits` parts: at M = 1024, K = 8192
// the 256 x 256 tiles number only 128, so the unsplit path uses 256 x 128
// tiles (one per CU), which run at ~0.65x the 256 x 256 tile's rate; two
// splits give 256 workgroups of 256 x 256 tiles.  With fewer tokens the
// unsplit kernel leaves most CUs idle (M = 128, K = 4096: 32 workgroups).  Each split stores an FP32
// partial dX into the workspace ([split][M][K4], K4 = K rounded up to 4), and
// splitk_reduce adds them in split order -- deterministic, but a different
// summation order from the unsplit kernel.
// Output tiles of the split kernel: 256 x 256, or 256 x 128 for M <= 128.
int64_t dgrad_split_tiles(int64_t M, int64_t K)
{
    return ((K + 255) / 256) * (M <= 128 ? (M + 127) / 128 : (M + 255) / 256);
}

// Parts: enough for ~256 workgroups (a power of two, at most 16), each at
// least 2048 deep in V.  Measured on MI355X (same box): M=1024 K=8192 V=32768
// two parts, 0.61 -> 0.45 ms; M=512 four, 449 -> 266 us; M=256 eight, 447 ->
// 153 us; M=128 K=4096 sixteen, 370 -> 75 us; M=16 K=4096 sixteen, 306 -> 61
// us.  256 or more tiles run unsplit.
int dgrad_default_splits(int64_t M, int64_t K, int64_t V)
{
    const int64_t tiles = dgrad_split_tiles(M, K);
    int s = 1;
    while (s < 16 && tiles * s * 2 <= 256 && V / (s * 2) >= 2048)
        s *= 2;
    return s;
}

namespace {

int64_t split_len(int64_t P, int splits)
{
    const int64_t per = (P + splits - 1) / splits;
    return (per + 63) / 64 * 64;  // whole 64-deep stages
}

// out[c][r] = sum over z = 0 .. S-1 (in order) of ws[z][c][r], r < R, c < C;
// pitch R4 in ws.  Each thread takes 4 consecutive r of one row.
template <bool BF16>
__global__ void __launch_bounds__(256) splitk_reduce(const float *ws, int S, int64_t stride,
                                                     int64_t R, int64_t R4, int64_t C, void *D,
                                                     int64_t ldd)
{
    const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t per_row = R4 / 4;
    const int64_t c = q / per_row;
    const int64_t r = (q - c * per_row) * 4;
    if (c >= C)
        return;
    const float *src = ws + c * R4 + r;
    float4 a = *reinterpret_cast<const float4 *>(src);
    for (int z = 1; z < S; ++z) {
        const float4 b = *reinterpret_cast<const float4 *>(src + z * stride);
        a.x += b.x, a.y += b.y, a.z += b.z, a.w += b.w;
    }
    const float v[4] = {a.x, a.y, a.z, a.w};
    if constexpr (BF16) {
        uint16_t *out = static_cast<uint16_t *>(D) + c * ldd + r;
        const f32x2 lo = {a.x, a.y}, hi = {a.z, a.w};
        const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        if (r + 4 <= R) {
            store8(out, make_uint2(w0, w1), true);
        } else {
            const uint32_t w[2] = {w0, w1};
            for (int e = 0; e < 4 && r + e < R; ++e)
                out[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        }
    } else {
        float *out = static_cast<float *>(D) + c * ldd + r;
        if (r + 4 <= R) {
            store16(out, a, true);
        } else {
            for (int e = 0; e < 4 && r + e < R; ++e)
                out[e] = v[e];
        }
    }
}

}  // namespace

int64_t dgrad_workspace_elems(int64_t M, int64_t K, int64_t V, int splits)
{
    if (splits <= 0)
        splits = dgrad_default_splits(M, K, V);
    if (splits <= 1 || M <= 0 || K <= 0 || V <= 0)
        return 0;
    const int64_t ps = split_len(V, splits);
    const int64_t ns = (V + ps - 1) / ps;
    return ns * M * ((K + 3) / 4 * 4);
}

hipError_t launch_gemm_dgrad_split(const GemmProblem &p, bool bf16_out, int splits, float *ws,
                                   hipStream_t s)
{
    // p: R = K, C = M, P = V, D = dX (ldd), as for launch_gemm_dgrad.
    if (splits <= 0)
        splits = dgrad_default_splits(p.C, p.R, p.P);
    if (splits <= 1 || p.P <= 0 || p.R <= 0 || p.C <= 0 || !ws)
        return launch_gemm_dgrad(p, bf16_out ? Epi::kStoreBF16 : Epi::kStoreF32, s);
    const int64_t R4 = (p.R + 3) / 4 * 4;
    GemmProblem q = p;
    q.psplit = split_len(p.P, splits);
    q.split_stride = p.C * R4;
    q.D = ws;
    q.ldd = R4;
    q.stream_out = false;  // read back at once by splitk_reduce
    const int ns = static_cast<int>((p.P + q.psplit - 1) / q.psplit);
    if (!big_offsets_fit(q))
        return launch_gemm_dgrad(p, bf16_out ? Epi::kStoreBF16 : Epi::kStoreF32, s);
    // Tile order: 2 tile rows (K) walked before stepping along M, so the
    // tiles that share a W strip run on one XCD.  Measured on MI355X against
    // 8 (bitwise-identical dX, three alternated rounds of 15): M=512 K=8192
    // V=32768 261-318 -> 243-262 us, M=1024 452-519 -> 447-485, M=128 K=4096
    // 70.1-71.4 -> 68.2-69.8, M=512 K=16384 V=131072 1778-1804 -> 1766-1772,
    // M=256 within 1 %; 4 was within 1 % of 2, 16 slower.
    constexpr int kSplitGroup = 2;
    const hipError_t e =
        p.C <= 128 ? launch_big<256, 128, 4, 2, true, false>(q, Epi::kStoreF32, kSplitGroup, s)
                   : launch_big<256, 256, 4, 2, true, false>(q, Epi::kStoreF32, kSplitGroup, s);
    if (e != hipSuccess)
        return e;
    const int64_t nthr = p.C * (R4 / 4);
    const unsigned blocks = static_cast<unsigned>((nthr + 255) / 256);
    if (bf16_out)
        hipLaunchKernelGGL(splitk_reduce<true>, dim3(blocks), dim3(256), 0, s, ws, ns,
                           q.split_stride, p.R, R4, p.C, p.D, p.ldd);
    else
        hipLaunchKernelGGL(splitk_reduce<false>, dim3(blocks), dim3(256), 0, s, ws, ns,
                           q.split_stride, p.R, R4, p.C, p.D, p.ldd);
    return hipGetLastError();
}

hipError_t launch_gemm_wgrad(const GemmProblem &p, Epi epi, hipStream_t s)
{
    // R = K (hidden), C = V (vocabulary); both operands stored [M][*].
    return launch_bwd<true, true>(p, epi, s);
}

}  // namespace lmh
