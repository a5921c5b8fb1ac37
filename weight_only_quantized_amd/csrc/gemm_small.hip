// gemm_small.hip — decode-sized W4A16 GEMM (M <= 16, or M <= 64 with two
// 16-row tiles per workgroup and 32-row groups on the grid): split-K over the
// waves of a workgroup, reduced through LDS.
//
// Work split: a workgroup owns NB 16-column blocks and the whole K range.
// Wave w owns the K slice of SG consecutive 128-row groups w*SG .. w*SG+SG-1
// for every one of the NB blocks, so it loads its slice of x once (SG x 64
// bytes per lane) and reuses it for all blocks.  Its NB*SG weight tiles
// (1 KB each, one 128-bit load per lane) are streamed through a software
// pipeline D tiles deep: the load of tile q+D is issued before tile q is
// multiplied, and scheduling barriers keep the compiler from hoisting the
// later loads, so the memory system always holds D tiles per wave while the
// wave computes.  Every load is unconditional (clamped row / group indices):
// a branch around a load forces a wait for all outstanding loads.
//
// Per group a wave dequantizes each lane's 32 nibbles in registers and runs
// 16x16x32 matrix-core steps with x padded to 16 rows; the per-group scale is
// applied to the fp32 group sum (exact integer weights inside the matrix
// core) and the waves' partial sums are added in LDS and rounded once.
//
// Matrix-core operand mapping (v_mfma_f32_16x16x32_{bf16,f16}): lane l feeds
// row/column l % 16 and k-block l / 16.  The weight slot of lane l holds
// column l % 16, rows 32*(l/16) + 0..31, so step t feeds rows 32*(l/16) + 8t + i
// for both operands.  The result register r of lane l is row 4*(l/16) + r,
// column l % 16.
//
// bf16 bias removal: the dequantized operand is 128 + v.  Per group, four
// extra steps with B = 1.0 in every slot give the row sums S of x; each tile
// then adds -(128 + z) * S with one fused multiply-add per result register,
// leaving sum_k x * (v - z).  Without zero points z = 8 for every column, so
// the four extra steps use B = -136 and their result is the accumulator
// input of every block's chain.  fp16 subtracts (1024 + z) exactly with a
// packed fp16 add instead.
//
// Scales and zero points are fetched once per group for all NB blocks (one
// 16-bit and one 8-bit load per lane), packed as scale | bias << 16 (bias =
// 128 + z for bf16, z for fp16; scale 0 for a group past the end of K) and
// handed to the lanes that use them with a cross-lane permute; per tile a
// wave then issues a single memory instruction, the 128-bit weight load, as
// a buffer load whose tile offset is a scalar register (no per-load address
// arithmetic in the vector ALU).
//
// Scale groups of 32 or 64 rows (GS = 32 or 64; weights in the group-aligned
// layout, word t of slot L holding rows 32*t + 8*(L/16) + i): step t of a
// tile then multiplies the 32 consecutive rows 32t .. 32t + 31, which lie in
// one scale group, so each scale group's steps form their own chain and its
// scale (and zero point) applies to that chain's fp32 sum.  Lane l's A operand
// for step t is x[row][32t + 8*(l/16) + 0..7] accordingly.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int kSmallMaxWaves = 16;
// MT = 2 (two 16-row tiles: twice the x slice in registers) runs at most 8
// waves per workgroup (two per SIMD, 256 registers each)
constexpr int kSmallMaxWaves2 = 8;

// MT 16-row tiles of x share every dequantized weight operand.
template <int DT, bool ZERO, int NB, int SG, int D, int MT = 1, int GS = 0>
__global__ void __launch_bounds__((MT == 1 ? kSmallMaxWaves : kSmallMaxWaves2) * 64)
gemm_small_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp,
                  const uint16_t *__restrict__ scale, const uint8_t *__restrict__ zero,
                  uint16_t *__restrict__ y, int M, int64_t K, int64_t N, int gm, const float *__restrict__ cs,
                  const float *__restrict__ cz) {
    static_assert(NB == 1 || NB == 2 || NB == 4, "one 64-lane load covers the scales of <= 4 blocks");
    static_assert(MT == 1 || MT == 2, "one or two 16-row tiles");
    static_assert(GS == 0 || GS == 32 || GS == 64, "standard layout, or 32/64-row scale groups");
    constexpr int NSUB = GS ? kGroup / GS : 1;    // scale groups per 128-row tile
    constexpr int TSUB = 4 / NSUB;                // matrix-core steps per scale group
    constexpr int T = NB * SG;                    // tiles per wave, ordered block-major
    const int G = (int)(K / kGroup);
    const int W = blockDim.x >> 6;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;       // row of the A operand / column of B and D
    const int kc = lane >> 4;      // 32-row chunk within a group
    const int64_t nb0 = (int64_t)blockIdx.x * NB;
    const int g0 = wave * SG;
    // two-tile form: 32-row groups of x on the second grid axis (each streams
    // the weights; the row groups of a column block share one XCD's L2)
    const int m0 = MT == 1 ? 0 : (int)blockIdx.y * 16 * MT;

    // Rows >= M read row M - 1 (in bounds, finite): the matrix core keeps rows
    // apart, and those result rows are never stored.  No branch around the
    // loads, so no wait for every outstanding load.
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(x);
    uint32_t xoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int jrow = m0 + 16 * mt + j < M ? m0 + 16 * mt + j : M - 1;
        xoff[mt] = (uint32_t)((int64_t)jrow * K + (GS ? 8 : 32) * kc) * 2u;
    }
    // buffer resource over this workgroup's NB * G weight tiles (raw, 32-bit
    // data format; every offset below is in range)
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wp + nb0 * G * kTileBytes), (short)0, NB * G * kTileBytes, 0x00020000);
    const int woff = lane * 16;

    // ---- x slice of this wave: A operands of every group, loaded once ---------
    u32x4_t xa[SG][MT][4];
#pragma unroll
    for (int i = 0; i < SG; ++i) {
        const int g = g0 + i < G ? g0 + i : G - 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xa[i][mt][t] = ld128(xbase + (int64_t)g * (kGroup * 2) + xoff[mt] + (GS ? 64 : 16) * t);
    }

    // ---- scales and zero points: one load per group for all NB blocks -------
    // Lane l fetches column 16*nb0 + l % (16*NB) and keeps scale | bias << 16;
    // the lane that multiplies block b fetches it from lane 16*b + j with a
    // cross-lane permute (no memory access) when the tile is reached.  A group
    // past the end of K (G not a multiple of SG) gets scale 0: its clamped,
    // finite tile then contributes nothing.
    constexpr uint32_t kBiasBase = DT == DT_BF16 ? 128u : 0u;
    uint32_t sz[SG][NSUB];
    {
        const int cl = lane & (16 * NB - 1);
        const int64_t col = nb0 * 16 + cl;
#pragma unroll
        for (int i = 0; i < SG; ++i)
#pragma unroll
            for (int h = 0; h < NSUB; ++h) {
                const bool live = g0 + i < G;
                const int g = live ? g0 + i : G - 1;
                // scale group: gm 128-row tiles each, or NSUB per tile
                const int64_t gs = GS ? (int64_t)g * NSUB + h : g / gm;
                const uint32_t sbits = scale[gs * N + col];
                uint32_t zb = 8u;
                if constexpr (ZERO) zb = __builtin_amdgcn_ubfe(zero[(gs * N + col) >> 1], (uint32_t)(cl & 1) * 4u, 4);
                sz[i][h] = (live ? sbits : 0u) | (kBiasBase + zb) << 16;
            }
    }

    // ---- weight tile stream ---------------------------------------------------
    u32x4_t raw[T];
    auto issue = [&](int q) {
        const int b = q / SG, i = q % SG;
        const int g = g0 + i < G ? g0 + i : G - 1;
        raw[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, woff, (b * G + g) * kTileBytes, 0));
    };
#pragma unroll
    for (int q = 0; q < D && q < T; ++q) issue(q);

    // bf16: per group either the bias chain of signed weights (-136 * row sum,
    // the same for every block, used as accumulator input) or, with zero
    // points, the row sums of x (B = 1.0 in every slot) that each tile scales
    // by its column's -(128 + z).
    // (per scale group of the tile: one chain of TSUB steps each)
    f32x4_t corr[SG][MT][NSUB];
    if constexpr (DT == DT_BF16) {
        const uint32_t c2 = ZERO ? 0x3F803F80u : bf16_negbias(8) * 0x10001u;
        const u32x4_t bc = {c2, c2, c2, c2};
#pragma unroll
        for (int i = 0; i < SG; ++i)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int h = 0; h < NSUB; ++h) {
                    corr[i][mt][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = h * TSUB; t < (h + 1) * TSUB; ++t)
                        corr[i][mt][h] = mfma16x16x32<DT>(xa[i][mt][t], bc, corr[i][mt][h]);
                }
    }

    float yacc[NB][MT][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[b][mt][r] = 0.f;

#pragma unroll
    for (int q = 0; q < T; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        if (q + D < T) issue(q + D);
        __builtin_amdgcn_sched_barrier(0);
        const int b = q / SG, i = q % SG;
#pragma unroll
        for (int h = 0; h < NSUB; ++h) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * b + j) << 2, (int)sz[i][h]);
            f32x4_t acc[MT];
            uint32_t nb2 = 0;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (DT == DT_BF16 && !ZERO) acc[mt] = corr[i][mt][h];
                else acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            if constexpr (DT == DT_F16) nb2 = ZERO ? f16_negbias2(v >> 16) : f16_negbias2(8u);
#pragma unroll
            for (int t = h * TSUB; t < (h + 1) * TSUB; ++t) {
                const u32x4_t wq = dequant_word<DT>(raw[q][t], nb2);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16x16x32<DT>(xa[i][mt][t], wq, acc[mt]);
            }
            if constexpr (DT == DT_BF16 && ZERO) {
                // 128 + z sits in byte 2: one byte-to-float conversion
                const float nbias = -(float)((v >> 16) & 0xFFu);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt][r] = __builtin_fmaf(nbias, corr[i][mt][h][r], acc[mt][r]);
            }
            const float sv = h2f<DT>((uint16_t)(v & 0xFFFFu));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) yacc[b][mt][r] += sv * acc[mt][r];
        }
    }

    // ---- reduce the waves' partial sums ---------------------------------------
    __shared__ float red[MT == 1 ? kSmallMaxWaves : kSmallMaxWaves2][NB][16 * MT][17];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][b][16 * mt + 4 * kc + r][j] = yacc[b][mt][r];
    __syncthreads();

    for (int idx = threadIdx.x; idx < NB * 256 * MT; idx += W * 64) {
        const int b = idx / (256 * MT), row = (idx >> 4) % (16 * MT), col = idx & 15;
        if (m0 + row < M) {
            float sum = 0.f;
            for (int w = 0; w < W; ++w) sum += red[w][b][row][col];
            if (cz) sum -= cz[(int64_t)(m0 + row) * N + (nb0 + b) * 16 + col];   // floating-point zero points
            if (cs) sum *= cs[(nb0 + b) * 16 + col];     // secondary (per-column) scale
            y[(int64_t)(m0 + row) * N + (nb0 + b) * 16 + col] = f2h<DT>(sum);
        }
    }
}

// Variant table for the small-M kernel: (NB, SG, D).  Index 0 is the default
// for every M <= 16 (at K = 4096, N = 14336 it beats index 1, every tile of a
// wave in flight at once, by 0.2-0.3 us at M = 2..16); the others are kept for
// tuning through the test hook.
struct SmallCfg { int nb, sg, d; };
static constexpr SmallCfg kSmallCfgs[] = {{4, 2, 4}, {4, 2, 8}, {4, 2, 2}, {2, 4, 4}, {2, 2, 4},
                                          {1, 2, 2}, {1, 4, 4}, {4, 1, 4}};
static std::atomic<int> g_small_cfg{-1};     // -1: automatic

int small_config_count() { return (int)(sizeof(kSmallCfgs) / sizeof(kSmallCfgs[0])); }
void set_small_config(int idx) { g_small_cfg.store(idx, std::memory_order_relaxed); }
int64_t small_max_k() { return (int64_t)kSmallMaxWaves * 4 * kGroup; }

template <int DT, bool ZERO, int NB, int SG, int D, int MT = 1, int GS = 0>
static hipError_t small_launch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                               int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                               hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t waves = (G + SG - 1) / SG;
    const dim3 grid((unsigned)(N / (16 * NB)), MT == 1 ? 1u : (unsigned)((M + 16 * MT - 1) / (16 * MT)));
    hipLaunchKernelGGL((gemm_small_kernel<DT, ZERO, NB, SG, D, MT, GS>), grid, dim3((unsigned)(waves * 64)), 0, stream,
                       (const uint16_t *)x, (const uint8_t *)wp, (const uint16_t *)scale,
                       (const uint8_t *)zero, (uint16_t *)y, (int)M, K, N, gm, cs, cz);
    return hipGetLastError();
}

template <int DT, bool ZERO>
static hipError_t small_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                 int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                                 hipStream_t stream) {
    const int64_t G = K / kGroup;
    int idx = g_small_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= small_config_count()) idx = 0;
    SmallCfg c = kSmallCfgs[idx];
    // at most 16 waves per workgroup: widen the per-wave slice for long K, and
    // keep NB * SG <= 8 and D <= NB * SG so the tile pipeline and x slice fit
    // in registers
    while ((G + c.sg - 1) / c.sg > kSmallMaxWaves && c.sg < 4) c.sg *= 2;
    if ((G + c.sg - 1) / c.sg > kSmallMaxWaves) return hipErrorInvalidValue;   // K > small_max_k()
    while (c.nb * c.sg > 8) c.nb /= 2;
    if (c.d > c.nb * c.sg) c.d = c.nb * c.sg >= 4 ? 4 : 2;
    // N must be a multiple of 16*NB (N % 64 == 0 always allows NB <= 4)
    while ((N / 16) % c.nb != 0) c.nb /= 2;
#define W4_SMALL(NBV, SGV, DV)                                                                  \
    if (c.nb == NBV && c.sg == SGV && c.d == DV)                                                \
        return small_launch<DT, ZERO, NBV, SGV, DV>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    W4_SMALL(4, 2, 4) W4_SMALL(4, 2, 8) W4_SMALL(4, 2, 2) W4_SMALL(2, 4, 4) W4_SMALL(2, 2, 4)
    W4_SMALL(2, 4, 8) W4_SMALL(1, 2, 2) W4_SMALL(1, 4, 4) W4_SMALL(2, 2, 2) W4_SMALL(2, 4, 2)
    W4_SMALL(1, 4, 2) W4_SMALL(1, 2, 4) W4_SMALL(4, 1, 4) W4_SMALL(2, 1, 4) W4_SMALL(1, 1, 4)
    W4_SMALL(1, 1, 2) W4_SMALL(2, 1, 2) W4_SMALL(4, 4, 4) W4_SMALL(4, 4, 8) W4_SMALL(2, 2, 8)
    W4_SMALL(1, 4, 8) W4_SMALL(4, 1, 2)
#undef W4_SMALL
    return hipErrorInvalidValue;
}

// Two 16-row tiles (16 < M <= 64 with K <= 4096; above 32 rows further
// 32-row groups on the grid): at most 8 waves, so SG = ceil(G / 8) in
// {1, 2, 4}, NB * SG <= 8 and every tile of a wave in flight.
int64_t small2_max_k() { return (int64_t)kSmallMaxWaves2 * 4 * kGroup; }

template <int DT, bool ZERO>
static hipError_t small2_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                  int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                                  hipStream_t stream) {
    const int64_t G = K / kGroup;
    if (G > kSmallMaxWaves2 * 4) return hipErrorInvalidValue;       // K > small2_max_k()
    const int sg = G <= kSmallMaxWaves2 ? 1 : G <= 2 * kSmallMaxWaves2 ? 2 : 4;
    int nb = 4;
    while ((N / 16) % nb != 0) nb /= 2;
#define W4_SMALL2(NBV, SGV, DV)                                                                 \
    if (nb == NBV && sg == SGV)                                                                 \
        return small_launch<DT, ZERO, NBV, SGV, DV, 2>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    W4_SMALL2(4, 4, 8) W4_SMALL2(2, 4, 8) W4_SMALL2(4, 2, 8) W4_SMALL2(4, 1, 4) W4_SMALL2(1, 4, 4) W4_SMALL2(2, 2, 4)
    W4_SMALL2(1, 2, 2) W4_SMALL2(2, 1, 2) W4_SMALL2(1, 1, 1)
#undef W4_SMALL2
    return hipErrorInvalidValue;
}

// Scale groups of 32 or 64 rows (group-aligned weights): one 16-row tile,
// K <= small_gs_max_k() (two groups per wave: with per-scale-group
// correction sums the x slice, tiles and sums of a wave stay within the 128
// registers a 16-wave workgroup allows), the default (NB, SG, D) by M; the
// tuning hook does not apply.
int64_t small_gs_max_k() { return (int64_t)kSmallMaxWaves * 2 * kGroup; }

template <int DT, bool ZERO, int GS>
static hipError_t small_gs_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                    int64_t M, int64_t K, int64_t N, const float *cs, const float *cz,
                                    hipStream_t stream) {
    if (M > 16 || K > small_gs_max_k()) return hipErrorInvalidValue;
    if (M > 4) return small_launch<DT, ZERO, 4, 2, 8, 1, GS>(x, wp, scale, zero, y, M, K, N, 1, cs, cz, stream);
    return small_launch<DT, ZERO, 4, 2, 4, 1, GS>(x, wp, scale, zero, y, M, K, N, 1, cs, cz, stream);
}

template <int GS>
static hipError_t small_gs_dispatch_dt(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                       int64_t M, int64_t K, int64_t N, int dt, const float *cs, const float *cz,
                                       hipStream_t stream) {
    if (dt == DT_BF16)
        return zero ? small_gs_dispatch<DT_BF16, true, GS>(x, wp, scale, zero, y, M, K, N, cs, cz, stream)
                    : small_gs_dispatch<DT_BF16, false, GS>(x, wp, scale, zero, y, M, K, N, cs, cz, stream);
    return zero ? small_gs_dispatch<DT_F16, true, GS>(x, wp, scale, zero, y, M, K, N, cs, cz, stream)
                : small_gs_dispatch<DT_F16, false, GS>(x, wp, scale, zero, y, M, K, N, cs, cz, stream);
}

hipError_t launch_gemm_small_gs(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                int64_t M, int64_t K, int64_t N, int dt, int group_size, hipStream_t stream,
                                const float *cs, const float *cz) {
    if (group_size == 32) return small_gs_dispatch_dt<32>(x, wp, scale, zero, y, M, K, N, dt, cs, cz, stream);
    if (group_size == 64) return small_gs_dispatch_dt<64>(x, wp, scale, zero, y, M, K, N, dt, cs, cz, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_small(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                             int64_t M, int64_t K, int64_t N, int dt, hipStream_t stream, int gm, const float *cs,
                             const float *cz) {
    if (M > 16) {
        if (dt == DT_BF16)
            return zero ? small2_dispatch<DT_BF16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                        : small2_dispatch<DT_BF16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
        return zero ? small2_dispatch<DT_F16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                    : small2_dispatch<DT_F16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    }
    if (dt == DT_BF16)
        return zero ? small_dispatch<DT_BF16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                    : small_dispatch<DT_BF16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    return zero ? small_dispatch<DT_F16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                : small_dispatch<DT_F16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
}

}  // namespace w4
