// gemm_small.hip — decode-sized W4A16 GEMM (M <= 16): split-K over the waves
// of a workgroup, reduced through LDS.
//
// Work split: a workgroup owns NB 16-column blocks and the whole K range; its
// W waves take the 128-row groups round-robin (wave w: g = w, w+W, ...), so at
// any moment the waves of one workgroup stream adjacent 1 KB weight tiles.
// Per group a wave issues one 128-bit load per lane per column block (32
// nibbles of one column), dequantizes in registers and runs 16x16x32
// matrix-core steps with x padded to 16 rows.  The per-group scale is applied
// to the fp32 group sum (exact integer weights inside the matrix core), then
// partial sums of the W waves are added in LDS and rounded once.
//
// Matrix-core operand mapping (v_mfma_f32_16x16x32_{bf16,f16}): lane l feeds
// row/column l % 16 and k-block l / 16.  The weight slot of lane l holds
// column l % 16, rows 32*(l/16) + 0..31, so step t feeds rows 32*(l/16) + 8t + i
// for both operands.  The result register r of lane l is row 4*(l/16) + r,
// column l % 16.
//
// bf16 bias removal: the operand holds 128 + v; one extra 16x16x32 step with
// A = (hi, mid, lo) bf16 limbs of the row's group sum sum_k x[m][k] and
// B = -(128 + z) in three k slots subtracts (128 + z) * sum_k x exactly enough
// (24-bit sum, exact 16-bit products) before the scale is applied.
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

template <int DT, bool ZERO, int NB, int W>
__global__ void __launch_bounds__(W * 64)
gemm_small_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp,
                  const uint16_t *__restrict__ scale, const uint8_t *__restrict__ zero,
                  uint16_t *__restrict__ y, int M, int64_t K, int64_t N) {
    const int G = (int)(K / kGroup);
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;       // row of the A operand / column of B and D
    const int kc = lane >> 4;      // 32-row chunk within a group
    const int64_t nb0 = (int64_t)blockIdx.x * NB;

    float yacc[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[b][r] = 0.f;

    const bool row_ok = j < M;
    const uint16_t *xrow = x + (int64_t)j * K + 32 * kc;
    const uint8_t *wlane = wp + lane * 16;

    for (int g = wave; g < G; g += W) {
        u32x4_t raw[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) raw[b] = ld128(wlane + ((nb0 + b) * G + g) * kTileBytes);

        float s[NB];
        uint32_t z[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int64_t col = (nb0 + b) * 16 + j;
            s[b] = h2f<DT>(scale[(int64_t)g * N + col]);
            if constexpr (ZERO) {
                const uint8_t zb = zero[((int64_t)g * N + col) >> 1];
                z[b] = (col & 1) ? (zb >> 4) : (zb & 0xF);
            } else {
                z[b] = 8;          // signed weights are stored as q + 8
            }
        }

        u32x4_t xa[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (row_ok) xa[t] = ld128(xrow + (int64_t)g * kGroup + 8 * t);
            else xa[t] = u32x4_t{0, 0, 0, 0};
        }

        u32x4_t acorr = {0, 0, 0, 0};
        if constexpr (DT == DT_BF16) {
            const bf16x2_t ones = as<bf16x2_t>(0x3F803F80u);
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    ps = __builtin_amdgcn_fdot2_f32_bf16(as<bf16x2_t>(xa[t][p]), ones, ps, false);
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            if (kc == 0) {
                uint32_t hi, mid, lo;
                split3_bf16(ps, hi, mid, lo);
                acorr[0] = hi | (mid << 16);
                acorr[1] = lo;
            }
        }

#pragma unroll
        for (int b = 0; b < NB; ++b) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            uint32_t nb2 = 0;
            if constexpr (DT == DT_BF16) {
                u32x4_t bcorr = {0, 0, 0, 0};
                if (kc == 0) {
                    const uint32_t c = bf16_negbias(z[b]);
                    bcorr[0] = c | (c << 16);
                    bcorr[1] = c;
                }
                acc = mfma16x16x32<DT>(acorr, bcorr, acc);
            } else {
                nb2 = f16_negbias2(z[b]);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) acc = mfma16x16x32<DT>(xa[t], dequant_word<DT>(raw[b][t], nb2), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[b][r] += s[b] * acc[r];
        }
    }

    __shared__ float red[W][NB][16][17];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][b][4 * kc + r][j] = yacc[b][r];
    __syncthreads();

    for (int idx = threadIdx.x; idx < NB * 256; idx += W * 64) {
        const int b = idx >> 8, row = (idx >> 4) & 15, col = idx & 15;
        if (row < M) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) sum += red[w][b][row][col];
            y[(int64_t)row * N + (nb0 + b) * 16 + col] = f2h<DT>(sum);
        }
    }
}

template <int DT, bool ZERO>
static hipError_t small_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                 int64_t M, int64_t K, int64_t N, hipStream_t stream) {
    constexpr int NB = 2, W = 8;
    const dim3 grid((unsigned)(N / (16 * NB)));
    hipLaunchKernelGGL((gemm_small_kernel<DT, ZERO, NB, W>), grid, dim3(W * 64), 0, stream,
                       (const uint16_t *)x, (const uint8_t *)wp, (const uint16_t *)scale,
                       (const uint8_t *)zero, (uint16_t *)y, (int)M, K, N);
    return hipGetLastError();
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
