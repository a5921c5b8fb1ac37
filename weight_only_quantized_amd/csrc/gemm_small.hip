// gemm_small.hip — decode-sized W4A16 GEMM (M <= 16): split-K over the waves
// of a workgroup, reduced through LDS.
//
// Work split: a workgroup owns NB 16-column blocks and the whole K range; wave
// w owns the GW consecutive 128-row groups w*GW .. w*GW+GW-1, so for every
// column block its weight tiles are GW consecutive kilobytes.  The kernel is
// bound by HBM bandwidth, so each wave first issues every load it will need
// (NB*GW 128-bit weight loads per lane, the scales, zero points and x rows)
// and only then computes: the whole weight stream is in flight at once instead
// of one group's worth per round trip.
//
// Per group a wave dequantizes each lane's 32 nibbles in registers and runs
// 16x16x32 matrix-core steps with x padded to 16 rows.  The per-group scale is
// applied to the fp32 group sum (exact integer weights inside the matrix
// core), then the partial sums of the waves are added in LDS and rounded once.
//
// Matrix-core operand mapping (v_mfma_f32_16x16x32_{bf16,f16}): lane l feeds
// row/column l % 16 and k-block l / 16.  The weight slot of lane l holds
// column l % 16, rows 32*(l/16) + 0..31, so step t feeds rows 32*(l/16) + 8t + i
// for both operands.  The result register r of lane l is row 4*(l/16) + r,
// column l % 16.
//
// bf16 bias removal: the operand holds 128 + v; one extra 16x16x16 step with
// A = (hi, mid, lo) bf16 limbs of the row's group sum sum_k x[m][k] (three k
// slots of k-block 0, zero elsewhere) and B = -(128 + z) subtracts
// (128 + z) * sum_k x (24-bit sum, exact 16-bit products) before the scale is
// applied.
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int kSmallMaxWaves = 16;

template <int DT, bool ZERO, int NB, int GW>
__global__ void __launch_bounds__(kSmallMaxWaves * 64)
gemm_small_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp,
                  const uint16_t *__restrict__ scale, const uint8_t *__restrict__ zero,
                  uint16_t *__restrict__ y, int M, int64_t K, int64_t N) {
    const int G = (int)(K / kGroup);
    const int W = blockDim.x >> 6;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;       // row of the A operand / column of B and D
    const int kc = lane >> 4;      // 32-row chunk within a group
    const int64_t nb0 = (int64_t)blockIdx.x * NB;
    const int g0 = wave * GW;

    // Wave-uniform base addresses with 32-bit per-lane offsets, so every load
    // is a scalar-base + vector-offset access without 64-bit address math.
    // Loads are unconditional: A-operand rows >= M read row M-1 (they only feed
    // result rows that are never stored), and a group index past the end is
    // clamped to the last group with its scale forced to 0.
    const int jrow = j < M ? j : M - 1;
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(x);
    const uint32_t xoff = (uint32_t)((int64_t)jrow * K + 32 * kc) * 2u;
    const uint8_t *wblk = wp + nb0 * G * kTileBytes;
    const uint32_t woff = (uint32_t)lane * 16u;

    // ---- phase 1: issue every load of this wave (x first: the in-order load
    //      counter then never waits on weights it does not need yet) ----------
    u32x4_t xa[GW][4];
#pragma unroll
    for (int i = 0; i < GW; ++i) {
        const int g = g0 + i < G ? g0 + i : G - 1;
#pragma unroll
        for (int t = 0; t < 4; ++t) xa[i][t] = ld128(xbase + (int64_t)g * (kGroup * 2) + xoff + 16 * t);
    }
    u32x4_t raw[GW][NB];
#pragma unroll
    for (int i = 0; i < GW; ++i) {
        const int g = g0 + i < G ? g0 + i : G - 1;
#pragma unroll
        for (int b = 0; b < NB; ++b) raw[i][b] = ld128(wblk + ((int64_t)b * G + g) * kTileBytes + woff);
    }
    uint32_t sbits[GW][NB], zbyte[GW][NB];
#pragma unroll
    for (int i = 0; i < GW; ++i) {
        const bool live = g0 + i < G;
        const int g = live ? g0 + i : G - 1;
        const uint16_t *srow = scale + (int64_t)g * N + nb0 * 16;
        const uint8_t *zrow = ZERO ? zero + (((int64_t)g * N + nb0 * 16) >> 1) : nullptr;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            sbits[i][b] = live ? (uint32_t)srow[b * 16 + j] : 0u;
            zbyte[i][b] = ZERO ? (uint32_t)zrow[b * 8 + (j >> 1)] : 0u;
        }
    }

    // ---- phase 2: dequantize and multiply ------------------------------------
    float yacc[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[b][r] = 0.f;

    const uint32_t kc0 = kc == 0 ? 0xFFFFFFFFu : 0u;      // correction slots live in k-block 0
    const uint32_t zshift = (uint32_t)(j & 1) * 4u;        // nibble of this lane's column

#pragma unroll
    for (int i = 0; i < GW; ++i) {
        u32x2_t acorr = {0, 0};
        if constexpr (DT == DT_BF16) {
            const bf16x2_t ones = as<bf16x2_t>(0x3F803F80u);
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    ps = __builtin_amdgcn_fdot2_f32_bf16(as<bf16x2_t>(xa[i][t][p]), ones, ps, false);
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            uint32_t hi, mid, lo;
            split3_bf16(ps, hi, mid, lo);
            acorr[0] = (hi | (mid << 16)) & kc0;
            acorr[1] = lo & kc0;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t z = ZERO ? __builtin_amdgcn_ubfe(zbyte[i][b], zshift, 4) : 8u;
            f32x4_t acc;
            uint32_t nb2 = 0;
            if constexpr (DT == DT_BF16) {
                // lanes outside k-block 0 carry A = 0, so B needs no masking
                const uint32_t c = bf16_negbias(z);
                const u32x2_t bcorr = {c | (c << 16), c};
                acc = mfma16x16x16_bf16(acorr, bcorr, f32x4_t{0.f, 0.f, 0.f, 0.f});
            } else {
                nb2 = f16_negbias2(z);
                acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) acc = mfma16x16x32<DT>(xa[i][t], dequant_word<DT>(raw[i][b][t], nb2), acc);
            const float sv = h2f<DT>((uint16_t)sbits[i][b]);
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[b][r] += sv * acc[r];
        }
    }

    // ---- phase 3: reduce the waves' partial sums -------------------------------
    __shared__ float red[kSmallMaxWaves][NB][16][17];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][b][4 * kc + r][j] = yacc[b][r];
    __syncthreads();

    for (int idx = threadIdx.x; idx < NB * 256; idx += W * 64) {
        const int b = idx >> 8, row = (idx >> 4) & 15, col = idx & 15;
        if (row < M) {
            float sum = 0.f;
            for (int w = 0; w < W; ++w) sum += red[w][b][row][col];
            y[(int64_t)row * N + (nb0 + b) * 16 + col] = f2h<DT>(sum);
        }
    }
}

// Variant table for the small-M kernel: (NB, GW).  Index 0 is the default;
// the others are kept for tuning through the test hook.
struct SmallCfg { int nb, gw; };
static constexpr SmallCfg kSmallCfgs[] = {{2, 4}, {1, 4}, {4, 4}, {1, 2}, {2, 2}, {4, 2}, {1, 8}, {2, 8}};
static int g_small_cfg = -1;     // -1: automatic

int small_config_count() { return (int)(sizeof(kSmallCfgs) / sizeof(kSmallCfgs[0])); }
void set_small_config(int idx) { g_small_cfg = idx; }
int64_t small_max_k() { return (int64_t)kSmallMaxWaves * 8 * kGroup; }

template <int DT, bool ZERO, int NB, int GW>
static hipError_t small_launch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                               int64_t M, int64_t K, int64_t N, hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t waves = (G + GW - 1) / GW;
    const dim3 grid((unsigned)(N / (16 * NB)));
    hipLaunchKernelGGL((gemm_small_kernel<DT, ZERO, NB, GW>), grid, dim3((unsigned)(waves * 64)), 0, stream,
                       (const uint16_t *)x, (const uint8_t *)wp, (const uint16_t *)scale,
                       (const uint8_t *)zero, (uint16_t *)y, (int)M, K, N);
    return hipGetLastError();
}

template <int DT, bool ZERO>
static hipError_t small_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                 int64_t M, int64_t K, int64_t N, hipStream_t stream) {
    const int64_t G = K / kGroup;
    int idx = g_small_cfg;
    if (idx < 0 || idx >= small_config_count()) idx = 0;
    SmallCfg c = kSmallCfgs[idx];
    // at most 16 waves per workgroup: widen the per-wave group count for long K
    while ((G + c.gw - 1) / c.gw > kSmallMaxWaves && c.gw < 8) c.gw *= 2;
    if (c.gw == 8 && c.nb > 2) c.nb = 2;
    if ((G + c.gw - 1) / c.gw > kSmallMaxWaves) return hipErrorInvalidValue;  // K > small_max_k()
#define W4_SMALL(NBV, GWV)                                                                    \
    if (c.nb == NBV && c.gw == GWV)                                                           \
        return small_launch<DT, ZERO, NBV, GWV>(x, wp, scale, zero, y, M, K, N, stream);
    W4_SMALL(1, 2) W4_SMALL(2, 2) W4_SMALL(4, 2)
    W4_SMALL(1, 4) W4_SMALL(2, 4) W4_SMALL(4, 4)
    W4_SMALL(1, 8) W4_SMALL(2, 8)
#undef W4_SMALL
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_small(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                             int64_t M, int64_t K, int64_t N, int dt, hipStream_t stream) {
    if (dt == DT_BF16)
        return zero ? small_dispatch<DT_BF16, true>(x, wp, scale, zero, y, M, K, N, stream)
                    : small_dispatch<DT_BF16, false>(x, wp, scale, zero, y, M, K, N, stream);
    return zero ? small_dispatch<DT_F16, true>(x, wp, scale, zero, y, M, K, N, stream)
                : small_dispatch<DT_F16, false>(x, wp, scale, zero, y, M, K, N, stream);
}

}  // namespace w4
