// w8.hip — W8A16: 8-bit integer weights with fp16/bf16 activations (the
// WNA16 setting of the Humming article's quantization descriptor with N = 8):
// dequant(W)[k][n] = (q - z[k/gs][n]) * s[k/gs][n], q int8 (no zero points)
// or uint8 with uint8 zero points, fp32 accumulation, one rounding.
//
// Prepacked tile: 2048 bytes per (16-column block, 128-row group), ordered
// (expert, block, group).  Slot L (32 bytes) holds column 16*nb + L%16, rows
// 128*g + 32*(L/16) + r as byte r, the stored code being u = q + 128 for
// signed weights and u itself otherwise.  Lane l of a 16x16x32 step feeds
// column l % 16 and rows 32*(l/16) + 8t + i of step t: two 128-bit loads give
// a lane its 32 codes of one group.
//
// Dequantization into the 16-bit operand:
//  * fp16: a code byte under the exponent byte 0x64 is exactly 1024 + u; one
//    packed fp16 add of -(1024 + z) gives the exact integer u - z (|u - z|
//    <= 255 < 2048).  One v_perm and one packed add per two weights.
//  * bf16: seven mantissa bits cannot hold an 8-bit code, so each byte is
//    converted to fp32 (exact) and the upper halves of two such values form a
//    bf16 pair (exact: at most 8 significant bits).  The operand is u itself
//    and the zero point comes out through the row sums of x: acc - z * S,
//    S = sum_k x over the group (from extra matrix-core steps with B = 1, or
//    with B = -128 straight into the accumulator for signed weights).
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int kW8TileBytes = 2048;

// Eight codes (two words: rows i = 0..3 and 4..7) as the 16-bit operand of
// one 16x16x32 or 32x32x16 step (register p holds rows 2p, 2p + 1).
template <int DT>
__device__ __forceinline__ u32x4_t w8_dequant(uint32_t w0, uint32_t w1, uint32_t negbias2) {
    u32x4_t r;
    if constexpr (DT == DT_F16) {
        // v_perm_b32 selector bytes: 0-3 pick bytes of the second source, 4-7 of the first
        r[0] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
        r[1] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
        r[2] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
        r[3] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
        const f16x2_t nb = as<f16x2_t>(negbias2);
#pragma unroll
        for (int p = 0; p < 4; ++p) r[p] = __builtin_bit_cast(uint32_t, as<f16x2_t>(r[p]) + nb);
    } else {
        (void)negbias2;
        const uint32_t ws[2] = {w0, w1};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w = ws[h];
            const uint32_t f0 = __float_as_uint((float)(w & 0xFFu));
            const uint32_t f1 = __float_as_uint((float)((w >> 8) & 0xFFu));
            const uint32_t f2 = __float_as_uint((float)((w >> 16) & 0xFFu));
            const uint32_t f3 = __float_as_uint((float)(w >> 24));
            r[2 * h] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
            r[2 * h + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
        }
    }
    return r;
}

// ---------------------------------------------------------------------------
// Prepack: one 64-thread workgroup per 2048-byte tile.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) w8_prepack_kernel(const uint8_t *__restrict__ w, uint8_t *__restrict__ out,
                                                        int64_t K, int64_t N, int is_signed) {
    const int64_t G = K / kGroup, NB = N / 16;
    const int64_t tile = blockIdx.x;                 // (e * NB + nb) * G + g
    const int64_t g = tile % G;
    const int64_t nb = (tile / G) % NB;
    const int64_t e = tile / (G * NB);
    const int L = threadIdx.x;

    __shared__ u32x4_t rows[kGroup];                  // 16 codes of each row
    const uint8_t *src = w + e * K * N + (g * kGroup) * N + nb * 16;
    for (int r = L; r < kGroup; r += 64) rows[r] = *reinterpret_cast<const u32x4_t *>(src + (int64_t)r * N);
    __syncthreads();

    const int h = L >> 4, j = L & 15;
    const uint32_t flip = is_signed ? 0x80808080u : 0u;   // q + 128 for two's complement q
    u32x4_t s0, s1;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t b = (rows[32 * h + 4 * d + i][j >> 2] >> (8 * (j & 3))) & 0xFFu;
            word |= b << (8 * i);
        }
        word ^= flip;
        if (d < 4) s0[d] = word; else s1[d - 4] = word;
    }
    uint8_t *dst = out + tile * kW8TileBytes + L * 32;
    *reinterpret_cast<u32x4_t *>(dst) = s0;
    *reinterpret_cast<u32x4_t *>(dst + 16) = s1;
}

// ---------------------------------------------------------------------------
// Small-M kernel (M <= 48, K <= 8192; one 16-row tile per grid row): the
// split-K structure of the W4A16 decode kernel.
// A workgroup owns NB 16-column blocks and all of K; wave w owns the SG groups
// w*SG .. w*SG+SG-1 for every block, loads its x slice once and streams its
// NB*SG tiles (two 128-bit buffer loads each) through a D-deep pipeline.
// ---------------------------------------------------------------------------
constexpr int kW8SmallMaxWaves = 16;

template <int DT, bool ZERO, int NB, int SG, int D>
__global__ void __launch_bounds__(kW8SmallMaxWaves * 64)
w8_small_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
                const uint8_t *__restrict__ zero, uint16_t *__restrict__ y, int M, int64_t K, int64_t N, int gm,
                const float *__restrict__ cs, const float *__restrict__ cz) {
    static_assert(NB == 1 || NB == 2 || NB == 4, "one 64-lane load covers the scales of <= 4 blocks");
    constexpr int T = NB * SG;
    const int G = (int)(K / kGroup);
    const int W = blockDim.x >> 6;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;
    const int kc = lane >> 4;
    const int64_t nb0 = (int64_t)blockIdx.x * NB;
    const int g0 = wave * SG;
    const int m0 = (int)blockIdx.y * 16;             // 16-row tile of x (grid rows)

    const int jrow = m0 + j < M ? m0 + j : M - 1;
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(x);
    const uint32_t xoff = (uint32_t)((int64_t)jrow * K + 32 * kc) * 2u;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wp + nb0 * G * kW8TileBytes), (short)0, NB * G * kW8TileBytes, 0x00020000);
    const int woff = lane * 32;

    u32x4_t xa[SG][4];
#pragma unroll
    for (int i = 0; i < SG; ++i) {
        const int g = g0 + i < G ? g0 + i : G - 1;
#pragma unroll
        for (int t = 0; t < 4; ++t) xa[i][t] = ld128(xbase + (int64_t)g * (kGroup * 2) + xoff + 16 * t);
    }

    // scale | zero << 16 for lane l's column 16*nb0 + l % (16*NB); scale 0 for a
    // group past the end of K
    uint32_t sz[SG];
    {
        const int cl = lane & (16 * NB - 1);
        const int64_t col = nb0 * 16 + cl;
#pragma unroll
        for (int i = 0; i < SG; ++i) {
            const bool live = g0 + i < G;
            const int g = live ? g0 + i : G - 1;
            const int64_t gs = g / gm;
            const uint32_t sbits = scale[gs * N + col];
            const uint32_t zb = ZERO ? (uint32_t)zero[gs * N + col] : 128u;
            sz[i] = (live ? sbits : 0u) | zb << 16;
        }
    }

    u32x4_t raw[T][2];
    auto issue = [&](int q) {
        const int b = q / SG, i = q % SG;
        const int g = g0 + i < G ? g0 + i : G - 1;
        const int toff = (b * G + g) * kW8TileBytes;
        raw[q][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, woff, toff, 0));
        raw[q][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, woff + 16, toff, 0));
    };
#pragma unroll
    for (int q = 0; q < D && q < T; ++q) issue(q);

    // bf16: row sums of x per group (B = 1.0), scaled per column by -z; for
    // signed weights (z = 128 everywhere) B = -128 gives the correction itself,
    // used as every block's accumulator input
    f32x4_t corr[SG];
    if constexpr (DT == DT_BF16) {
        const uint32_t c2 = ZERO ? 0x3F803F80u : 0xC300C300u;
        const u32x4_t bc = {c2, c2, c2, c2};
#pragma unroll
        for (int i = 0; i < SG; ++i) {
            corr[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) corr[i] = mfma16x16x32<DT>(xa[i][t], bc, corr[i]);
        }
    }

    float yacc[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[b][r] = 0.f;

#pragma unroll
    for (int q = 0; q < T; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        if (q + D < T) issue(q + D);
        __builtin_amdgcn_sched_barrier(0);
        const int b = q / SG, i = q % SG;
        const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * b + j) << 2, (int)sz[i]);
        f32x4_t acc;
        uint32_t nb2 = 0;
        if constexpr (DT == DT_BF16 && !ZERO) {
            acc = corr[i];
        } else {
            acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (DT == DT_F16) nb2 = f16_negbias2(v >> 16);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4_t &h = raw[q][t >> 1];
            const int d = 2 * (t & 1);
            acc = mfma16x16x32<DT>(xa[i][t], w8_dequant<DT>(h[d], h[d + 1], nb2), acc);
        }
        if constexpr (DT == DT_BF16 && ZERO) {
            const float nz = -(float)(v >> 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(nz, corr[i][r], acc[r]);
        }
        const float sv = h2f<DT>((uint16_t)(v & 0xFFFFu));
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[b][r] += sv * acc[r];
    }

    __shared__ float red[kW8SmallMaxWaves][NB][16][17];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][b][4 * kc + r][j] = yacc[b][r];
    __syncthreads();

    for (int idx = threadIdx.x; idx < NB * 256; idx += W * 64) {
        const int b = idx >> 8, row = (idx >> 4) & 15, col = idx & 15;
        if (m0 + row < M) {
            float sum = 0.f;
            for (int w = 0; w < W; ++w) sum += red[w][b][row][col];
            if (cz) sum -= cz[(int64_t)(m0 + row) * N + (nb0 + b) * 16 + col];   // floating-point zero points
            if (cs) sum *= cs[(nb0 + b) * 16 + col];     // secondary (per-column) scale
            y[(int64_t)(m0 + row) * N + (nb0 + b) * 16 + col] = f2h<DT>(sum);
        }
    }
}

// ---------------------------------------------------------------------------
// Tile kernel (M > 48, or K beyond the small kernel): the structure of the W4A16 tile kernel (x slice of a
// group staged in LDS, double-buffered, with the bf16 limbs of its row sums;
// weights straight from memory into registers; 32x32x16 steps; per-group
// scale on the fp32 group sum), with 8-bit weight fragments: four 128-bit
// loads per lane per 32 columns and group.
// ---------------------------------------------------------------------------
template <int DT, bool ZERO, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64, 2)
w8_tile_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
               const uint8_t *__restrict__ zero, uint16_t *__restrict__ y, int64_t M, int64_t K, int64_t N, int gm,
               const float *__restrict__ cs, const float *__restrict__ cz) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int RT = TM / 32, CT = TN / 32;
    constexpr bool CORR = DT == DT_BF16;
    constexpr int ROWB = (kGroup + (CORR ? 16 : 0)) * 2 + 16;
    constexpr int XP = BM * 16 / NT;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert((BM * 16) % NT == 0, "x staging must divide evenly");
    static_assert(XP <= 16, "one row-sum split per lane");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BM * ROWB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int G = (int)(K / kGroup);
    const int64_t row0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const bool wave_cols = n0 + (int64_t)wn * TN < N;
    const int64_t wcol0 = wave_cols ? n0 + (int64_t)wn * TN : N - TN;

    // ---- activation staging (rows past M read row M - 1, never stored) ------
    u32x4_t xr[XP];
    const uint16_t *xrow[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int id = p * NT + tid, r = id >> 4, c16 = id & 15;
        const int64_t grow = row0 + r < M ? row0 + r : M - 1;
        xrow[p] = x + grow * K + c16 * 8;
    }
    auto load_x = [&](int g) {
#pragma unroll
        for (int p = 0; p < XP; ++p) xr[p] = ld128(xrow[p] + (int64_t)g * kGroup);
    };
    auto row16_sum = [](float v) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
        return v;
    };
    auto store_x = [&](int buf) {
        uint8_t *base = lds + buf * BM * ROWB;
        float ps[XP];
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int id = p * NT + tid, r = id >> 4, c16 = id & 15;
            *reinterpret_cast<u32x4_t *>(base + r * ROWB + c16 * 16) = xr[p];
            if constexpr (CORR) {
                const bf16x2_t ones = as<bf16x2_t>(0x3F803F80u);
                float v = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v = __builtin_amdgcn_fdot2_f32_bf16(as<bf16x2_t>(xr[p][q]), ones, v, false);
                ps[p] = row16_sum(v);
            }
        }
        if constexpr (CORR) {
            const int c16 = tid & 15;
            float mine = ps[0];
#pragma unroll
            for (int p = 1; p < XP; ++p) mine = c16 == p ? ps[p] : mine;
            uint32_t hi, mid, lo;
            split3_bf16(mine, hi, mid, lo);
            if (c16 < XP) {
                const int r = (c16 * NT + tid) >> 4;
                *reinterpret_cast<u32x4_t *>(base + r * ROWB + 256) = u32x4_t{hi | (mid << 16), lo, 0, 0};
            }
        }
    };
    if constexpr (CORR) {
        for (int r = tid; r < 2 * BM; r += NT)
            *reinterpret_cast<u32x4_t *>(lds + r * ROWB + 272) = u32x4_t{0, 0, 0, 0};
    }

    // ---- weight fragments, scales and zero points ---------------------------
    // Lane l (column l % 32 of a 32-column tile, k-block kg = l / 32) needs
    // chunks 2*kg and 2*kg + 1 of its column's slot: 64 rows, 64 bytes.
    const int lj = lane & 31, kg = lane >> 5;
    int64_t boff[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int64_t n = wcol0 + ct * 32 + lj;
        boff[ct] = (n >> 4) * (int64_t)G * kW8TileBytes + ((2 * kg) * 16 + (n & 15)) * 32;
    }
    u32x4_t braw[CT][4], bnext[CT][4];
    uint16_t sraw[CT], snext[CT];
    uint8_t zraw[CT], znext[CT];
    auto load_b = [&](int g, u32x4_t (&dst)[CT][4], uint16_t (&sdst)[CT], uint8_t (&zdst)[CT]) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const uint8_t *p = wp + boff[ct] + (int64_t)g * kW8TileBytes;
            dst[ct][0] = ld128(p);
            dst[ct][1] = ld128(p + 16);
            dst[ct][2] = ld128(p + 512);           // chunk 2*kg + 1: 16 slots further
            dst[ct][3] = ld128(p + 528);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t n = wcol0 + ct * 32 + lj;
            const int64_t gs = g / gm;
            sdst[ct] = scale[gs * N + n];
            zdst[ct] = ZERO ? zero[gs * N + n] : (uint8_t)128;
        }
    };

    f32x16_t yacc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[rt][ct][r] = 0.f;

    load_x(0);
    load_b(0, braw, sraw, zraw);
    store_x(0);
    __syncthreads();

    const int arow = wm * TM + lj;
    auto step = [&](int g, const u32x4_t (&bw)[CT][4], const uint16_t (&sw)[CT], const uint8_t (&zw)[CT],
                    u32x4_t (&bn)[CT][4], uint16_t (&sn)[CT], uint8_t (&zn)[CT]) {
        const int buf = g & 1;
        const int gn = g + 1 < G ? g + 1 : g;
        load_x(gn);
        load_b(gn, bn, sn, zn);
        float s[CT];
        uint32_t nb2[CT];
        u32x4_t bcorr[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            s[ct] = h2f<DT>(sw[ct]);
            const uint32_t z = zw[ct];
            if constexpr (CORR) {
                const uint32_t c = bf16_bits_rne(-(float)z);   // exact: z <= 255
                bcorr[ct] = kg == 0 ? u32x4_t{c | (c << 16), c, 0, 0} : u32x4_t{0, 0, 0, 0};
                nb2[ct] = 0;
            } else {
                nb2[ct] = f16_negbias2(z);
            }
        }
        const uint8_t *abase = lds + buf * BM * ROWB + arow * ROWB + kg * 128;
        f32x16_t cin[RT][ZERO ? CT : 1];
        if constexpr (CORR) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t *>(
                    lds + buf * BM * ROWB + (arow + rt * 32) * ROWB + 256 + kg * 16);
#pragma unroll
                for (int ci = 0; ci < (ZERO ? CT : 1); ++ci) cin[rt][ci] = mfma32x32x16<DT>(a, bcorr[ci], f32x16_t{});
            }
        }
        f32x16_t acc[RT][CT];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            u32x4_t a[RT], bq[CT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                a[rt] = *reinterpret_cast<const u32x4_t *>(abase + rt * 32 * ROWB + t * 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                // step t: chunk t / 4, rows 8 (t % 4) .. + 7 = words 2 (t % 4), 2 (t % 4) + 1
                const u32x4_t &h = bw[ct][2 * (t >> 2) + ((t & 3) >> 1)];
                const int d = 2 * (t & 1);
                bq[ct] = w8_dequant<DT>(h[d], h[d + 1], nb2[ct]);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if (t == 0) {
                        if constexpr (CORR) acc[rt][ct] = mfma32x32x16<DT>(a[rt], bq[ct], cin[rt][ZERO ? ct : 0]);
                        else acc[rt][ct] = mfma32x32x16<DT>(a[rt], bq[ct], f32x16_t{});
                    } else {
                        acc[rt][ct] = mfma32x32x16<DT>(a[rt], bq[ct], acc[rt][ct]);
                    }
                }
            if (t == 4) store_x(buf ^ 1);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 16; ++r) yacc[rt][ct][r] += s[ct] * acc[rt][ct][r];
        __syncthreads();
    };
    for (int g = 0; g < G; g += 2) {
        step(g, braw, sraw, zraw, bnext, snext, znext);
        if (g + 1 < G) step(g + 1, bnext, snext, znext, braw, sraw, zraw);
    }

    if (!wave_cols) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t col = wcol0 + ct * 32 + lj;
            const float t = cs ? cs[col] : 1.f;           // secondary (per-column) scale
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = row0 + wm * TM + rt * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
                if (row < M) {
                    float v = yacc[rt][ct][r];
                    if (cz) v -= cz[row * N + col];       // floating-point zero points
                    y[row * N + col] = f2h<DT>(cs ? v * t : v);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
size_t w8_prepacked_bytes(int64_t E, int64_t K, int64_t N) { return (size_t)E * (size_t)K * (size_t)N; }

hipError_t launch_w8_prepack(const void *w, void *out, int64_t E, int64_t K, int64_t N, int is_signed,
                             hipStream_t stream) {
    const int64_t per = (K / kGroup) * (N / 16);
    for (int64_t e = 0; e < E; ++e)
        hipLaunchKernelGGL(w8_prepack_kernel, dim3((unsigned)per), dim3(64), 0, stream,
                           (const uint8_t *)w + e * K * N, (uint8_t *)out + e * per * kW8TileBytes, K, N, is_signed);
    return hipGetLastError();
}

int64_t w8_small_max_k() { return (int64_t)kW8SmallMaxWaves * 4 * kGroup; }

struct W8SmallCfg { int nb, sg, d; };
static constexpr W8SmallCfg kW8SmallCfgs[] = {{4, 2, 4}, {4, 2, 8}, {2, 2, 4}, {1, 4, 4}};
static std::atomic<int> g_w8_small_cfg{-1};
int w8_small_config_count() { return (int)(sizeof(kW8SmallCfgs) / sizeof(kW8SmallCfgs[0])); }
void set_w8_small_config(int idx) { g_w8_small_cfg.store(idx, std::memory_order_relaxed); }

template <int DT, bool ZERO, int NB, int SG, int D>
static hipError_t w8_small_launch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                  int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                                  hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t waves = (G + SG - 1) / SG;
    hipLaunchKernelGGL((w8_small_kernel<DT, ZERO, NB, SG, D>), dim3((unsigned)(N / (16 * NB)), (unsigned)((M + 15) / 16)),
                       dim3((unsigned)(waves * 64)), 0, stream, (const uint16_t *)x, (const uint8_t *)wp,
                       (const uint16_t *)scale, (const uint8_t *)zero, (uint16_t *)y, (int)M, K, N, gm, cs, cz);
    return hipGetLastError();
}

template <int DT, bool ZERO>
static hipError_t w8_small_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                    int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                                    hipStream_t stream) {
    const int64_t G = K / kGroup;
    int idx = g_w8_small_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= w8_small_config_count()) idx = 0;
    W8SmallCfg c = kW8SmallCfgs[idx];
    while ((G + c.sg - 1) / c.sg > kW8SmallMaxWaves && c.sg < 4) c.sg *= 2;
    if ((G + c.sg - 1) / c.sg > kW8SmallMaxWaves) return hipErrorInvalidValue;
    // registers: the x slice (16 per group) and the tiles in flight (8 per
    // tile) within 128 per lane: at most 8 tiles, one block when SG = 4
    while (c.nb * c.sg > 8 || (c.sg >= 4 && c.nb > 1)) c.nb /= 2;
    if (c.d > c.nb * c.sg) c.d = c.nb * c.sg >= 4 ? 4 : 2;
    while ((N / 16) % c.nb != 0) c.nb /= 2;
#define W4_W8S(NBV, SGV, DV)                                                                    \
    if (c.nb == NBV && c.sg == SGV && c.d == DV)                                                \
        return w8_small_launch<DT, ZERO, NBV, SGV, DV>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    W4_W8S(4, 2, 4) W4_W8S(4, 2, 8) W4_W8S(2, 2, 4) W4_W8S(1, 4, 4) W4_W8S(1, 2, 2) W4_W8S(2, 2, 2)
    W4_W8S(1, 4, 2) W4_W8S(4, 1, 4) W4_W8S(2, 1, 2) W4_W8S(1, 2, 4) W4_W8S(1, 1, 2) W4_W8S(2, 1, 4)
    W4_W8S(4, 1, 2) W4_W8S(2, 2, 8)
#undef W4_W8S
    return hipErrorInvalidValue;
}

// Tile variants (BM, BN, WM, WN).  Defaults: for bf16 above M = 64, 64 x 128
// with four 64 x 32 waves (the byte-to-bf16 conversion makes the kernel
// vector-ALU bound, and a 64-row wave tile converts each weight once for two
// row blocks: 4096^3 in 220-225 us against 252-254 us for 32 x 256 and
// 272-275 us for 64 x 128 with 32-row waves; 64 x 256 and 128 x 128 spill in
// bf16 and are not built there); 32 x 256 at M <= 64; for fp16 64 x 256 with
// four 64 x 64 waves.
struct W8TileCfg { int bm, bn, wm, wn; };
static constexpr W8TileCfg kW8TileCfgs[] = {{64, 256, 1, 4}, {32, 256, 1, 4}, {64, 128, 2, 2}, {64, 128, 1, 4},
                                            {128, 128, 1, 4}};
static std::atomic<int> g_w8_tile_cfg{-1};
int w8_tile_config_count() { return (int)(sizeof(kW8TileCfgs) / sizeof(kW8TileCfgs[0])); }
void set_w8_tile_config(int idx) { g_w8_tile_cfg.store(idx, std::memory_order_relaxed); }

template <int DT, bool ZERO, int BM, int BN, int WM, int WN>
static hipError_t w8_tile_launch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                 int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                                 hipStream_t stream) {
    if constexpr (DT == DT_BF16 && ((BM == 64 && BN == 256) || (BM == 128 && BN == 128))) {
        return hipErrorInvalidValue;             // not built: spills (see the table)
    } else {
        const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
        hipLaunchKernelGGL((w8_tile_kernel<DT, ZERO, BM, BN, WM, WN>), grid, dim3(WM * WN * 64), 0, stream,
                           (const uint16_t *)x, (const uint8_t *)wp, (const uint16_t *)scale, (const uint8_t *)zero,
                           (uint16_t *)y, M, K, N, gm, cs, cz);
        return hipGetLastError();
    }
}

template <int DT, bool ZERO>
static hipError_t w8_tile_dispatch(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                   int64_t M, int64_t K, int64_t N, int gm, const float *cs, const float *cz,
                                   hipStream_t stream) {
    int idx = g_w8_tile_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= w8_tile_config_count()) idx = M <= 64 ? 1 : (DT == DT_BF16 ? 3 : 0);
    if (DT == DT_BF16 && (idx == 0 || idx == 4)) idx = 3;
    const W8TileCfg c = kW8TileCfgs[idx];
#define W4_W8T(BMV, BNV, WMV, WNV)                                                              \
    if (c.bm == BMV && c.bn == BNV && c.wm == WMV && c.wn == WNV)                               \
        return w8_tile_launch<DT, ZERO, BMV, BNV, WMV, WNV>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    W4_W8T(64, 256, 1, 4) W4_W8T(32, 256, 1, 4) W4_W8T(64, 128, 2, 2) W4_W8T(64, 128, 1, 4) W4_W8T(128, 128, 1, 4)
#undef W4_W8T
    return hipErrorInvalidValue;
}

hipError_t launch_w8_gemm(const void *x, const void *wp, const void *scale, const void *zero, void *y, int64_t M,
                          int64_t K, int64_t N, int dt, int gm, bool small, hipStream_t stream, const float *cs,
                          const float *cz) {
    if (M == 0) return hipSuccess;
    if (small) {
        if (dt == DT_BF16)
            return zero ? w8_small_dispatch<DT_BF16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                        : w8_small_dispatch<DT_BF16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
        return zero ? w8_small_dispatch<DT_F16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                    : w8_small_dispatch<DT_F16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    }
    if (dt == DT_BF16)
        return zero ? w8_tile_dispatch<DT_BF16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                    : w8_tile_dispatch<DT_BF16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
    return zero ? w8_tile_dispatch<DT_F16, true>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream)
                : w8_tile_dispatch<DT_F16, false>(x, wp, scale, zero, y, M, K, N, gm, cs, cz, stream);
}

}  // namespace w4
