// msd.hip — MSD A16W4 PerGroup GEMM ("WeightQuantBatchMatmulExperiment
// operator deep-dive", §4.1 eqs. 1-11; pipeline of §6.1).
//
// Stage order follows the page's basic pipeline: pre-processing (A_max and the
// three residual layers) -> integer matmul -> post-processing (merge), with a
// device-wide sync between pre-processing and the matmul.  On the GPU that
// sync is the kernel boundary between msd_decompose_kernel and
// msd_gemm_kernel; the merge is fused into the matmul kernel's epilogue, so
// Y_int never leaves registers (the page's preload template overlaps the
// three stages across rounds, §6.2; here the waves of a compute unit overlap
// matrix-core products and vector merges of different groups).
//
// Workspace (caller-owned): coef [G][4][Mpad] fp32 (A_max / (7.49*14.98^j)
// for j = 0..2, then the code-bias term 8 * sum_j coef_j * S_j), layer sums
// S [G][3][Mpad] int32 (sum over the group of each layer), amax [M][G] fp32,
// layers [3][Mpad][K] int8 in operand order, and for K splits > 1 partial
// sums [ksplit][M][N] fp32.
//
// The weights enter the integer matrix core as their stored codes u = q + 8
// (0..15, no conversion to signed bytes): each layer's product is then
// Y'_j = Y_j + 8 * S_j, and the merge starts its chain from -8 * sum_j
// coef_j * S_j (one fused multiply-add absorbs it, the cancellation is exact
// inside the fma), so the merge costs no more than with signed operands.
//
// Layer storage order: inside each aligned 8-k block, byte p holds
// k = base + {0,4,1,5,2,6,3,7}[p].  That is the order in which the int8
// operand of the weights comes out of one prepacked word
// (word & 0x0F0F0F0F gives rows 0,4,1,5; (word >> 4) & 0x0F0F0F0F gives
// 2,6,3,7), so both operands of v_mfma_i32_16x16x64_i8 see the same k in the
// same byte.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

__device__ __forceinline__ int perm8(int p) { return ((p & 1) << 2) | (p >> 1); }   // {0,4,1,5,2,6,3,7}

// MSD factors (fp32 constants of the page, §4.1) and the merge reciprocals.
constexpr float kF1 = 7.49f;
constexpr float kF2 = 14.98f;
constexpr float kR0 = (float)(1.0 / (double)7.49f);
constexpr float kR1 = (float)(1.0 / ((double)7.49f * (double)14.98f));
constexpr float kR2 = (float)(1.0 / ((double)7.49f * (double)14.98f * (double)14.98f));

// eqs.2-7, one binary32 operation per line, no contraction, RNE rounding.
__device__ __forceinline__ void msd_decompose(float a, float amax, int &l1, int &l2, int &l3) {
#pragma clang fp contract(off)
    if (amax == 0.f) {
        l1 = l2 = l3 = 0;
        return;
    }
    const float t1 = (kF1 * a) / amax;         // tmp1 = 7.49*A/A_max (correctly rounded division)
    const float a1 = __builtin_rintf(t1);      // A1 = round(tmp1), half to even
    const float t2 = (t1 - a1) * kF2;          // tmp2 = (tmp1 - A1)*14.98
    const float a2 = __builtin_rintf(t2);
    const float t3 = (t2 - a2) * kF2;          // tmp3 = (tmp2 - A2)*14.98
    const float a3 = __builtin_rintf(t3);
    l1 = (int)a1;
    l2 = (int)a2;
    l3 = (int)a3;
}

// Sum and maximum over the 64 lanes of a wave with DPP moves (quad
// permutations, half-row and row mirrors, then the row broadcasts of lanes 15
// and 31), read from lane 63: a wave-uniform result without LDS round trips.
// Integer sums and maxima do not depend on the order of the operations; a
// lane whose DPP source is disabled combines with `fill`.
// The first four steps leave every lane of a 16-lane row with the row's
// result (row_reduce_dpp).
template <typename F>
__device__ __forceinline__ int row_reduce_dpp(int v, int fill, F op) {
    v = op(v, __builtin_amdgcn_update_dpp(fill, v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    v = op(v, __builtin_amdgcn_update_dpp(fill, v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    v = op(v, __builtin_amdgcn_update_dpp(fill, v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = op(v, __builtin_amdgcn_update_dpp(fill, v, 0x140, 0xF, 0xF, false));   // row_mirror
    return v;
}
template <typename F>
__device__ __forceinline__ int wave_reduce_dpp(int v, int fill, F op) {
    v = row_reduce_dpp(v, fill, op);
    v = op(v, __builtin_amdgcn_update_dpp(fill, v, 0x142, 0xA, 0xF, false));   // row_bcast:15 into rows 1, 3
    v = op(v, __builtin_amdgcn_update_dpp(fill, v, 0x143, 0xC, 0xF, false));   // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_sum_i32(int v) {
    return wave_reduce_dpp(v, 0, [](int a, int b) { return a + b; });
}
// maximum of non-negative floats with fmaxf, as in msd_decompose_kernel
// (rows left out of a broadcast keep their value: fmaxf(v, 0) for v >= 0)
__device__ __forceinline__ float wave_max_nonneg(float v) {
    return __builtin_bit_cast(float, wave_reduce_dpp(__builtin_bit_cast(int, v), 0, [](int a, int b) {
        return __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    }));
}

__device__ __forceinline__ int row_sum_i32(int v) {
    return row_reduce_dpp(v, 0, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ float row_max_nonneg(float v) {
    return __builtin_bit_cast(float, row_reduce_dpp(__builtin_bit_cast(int, v), 0, [](int a, int b) {
        return __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    }));
}

// One 256-thread workgroup handles 16 (row, group) pairs; 16 lanes (one DPP
// row) per pair, 8 elements per lane.
__global__ void __launch_bounds__(256)
msd_decompose_kernel(const uint16_t *__restrict__ x, float *__restrict__ coef, int32_t *__restrict__ lsum,
                     float *__restrict__ amax_out, int8_t *__restrict__ layers, int64_t M, int64_t Mpad,
                     int64_t K) {
    const int64_t G = K / kGroup;
    const int64_t pair = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    const int64_t m = pair / G, g = pair % G;
    const bool valid = pair < Mpad * G;
    const bool real = valid && m < M;

    u32x4_t v = {0, 0, 0, 0};
    if (real) v = ld128(x + m * K + g * kGroup + sub * 8);
    float a[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[2 * i] = h2f<DT_F16>((uint16_t)(v[i] & 0xFFFF));
        a[2 * i + 1] = h2f<DT_F16>((uint16_t)(v[i] >> 16));
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(a[i]));
    am = row_max_nonneg(am);                    // eq.1: A_max of the (row, group)
    if (!valid) return;

    int l[3][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) msd_decompose(a[i], am, l[0][i], l[1][i], l[2][i]);
    // layer sums over the group (16 lanes x 8 elements), exact in int32
    int ls[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        int t = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) t += l[j][i];
        ls[j] = row_sum_i32(t);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        uint64_t packed = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p) packed |= (uint64_t)(uint8_t)(int8_t)l[j][perm8(p)] << (8 * p);
        *reinterpret_cast<uint64_t *>(layers + (j * Mpad + m) * K + g * kGroup + sub * 8) = packed;
    }
    if (sub == 0) {
        const float c0 = am * kR0, c1 = am * kR1, c2 = am * kR2;
        coef[(g * 4 + 0) * Mpad + m] = c0;
        coef[(g * 4 + 1) * Mpad + m] = c1;
        coef[(g * 4 + 2) * Mpad + m] = c2;
        coef[(g * 4 + 3) * Mpad + m] =
            8.f * __builtin_fmaf(c0, (float)ls[0], __builtin_fmaf(c1, (float)ls[1], c2 * (float)ls[2]));
#pragma unroll
        for (int j = 0; j < 3; ++j) lsum[(g * 3 + j) * Mpad + m] = ls[j];
        if (real) amax_out[m * G + g] = am;
    }
}

// int8 operand of one 16x16x64 step from two prepacked words: the stored
// codes u = q + 8 (0..15), one per byte.
__device__ __forceinline__ u32x4_t weight_u4(uint32_t w0, uint32_t w1) {
    return u32x4_t{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
}

// Integer products of the three layers with the weights (eq.9) and the merge
// (eqs.10-11).
//
// A workgroup owns ROWS = 16*MT x rows, W*NB 16-column blocks (NB per wave)
// and one K slice of GPS groups (blockIdx.y; the last slice may hold fewer:
// its missing groups get zero coefficients).  The three layers of
// its rows over the whole slice and their merge coefficients are loaded into
// LDS once (one barrier); then every wave streams its own weight tiles with no
// further synchronisation: the tiles of group g + 2 are fetched while group g
// is multiplied (three register sets in a ring), every layer fragment read
// from LDS serves the wave's NB blocks, and every load is unconditional
// (clamped indices).  LDS rows are padded by 16 bytes so the 16 rows read by
// one operand load fall on disjoint banks.
//
// Lane l of v_mfma_i32_16x16x64_i8 feeds row/column l % 16 and k-block l / 16:
// the weight slot of lane l holds rows 32*(l/16) + 0..31 of the group, step s
// uses its words 2s, 2s+1 (rows 32*(l/16) + 16s + 0..15) and the layer bytes
// 32*(l/16) + 16s .. +15 of the same row order.  Result register r of lane l
// is row 4*(l/16) + r, column l % 16.
template <int MT> struct MsdLds {
    static constexpr int GPSMAX = MT == 1 ? 16 : MT == 2 ? 8 : 4;     // ~100 KB of layers
    static constexpr int ROWS = 16 * MT;
    static constexpr int AROW = GPSMAX * kGroup + 16;                  // LDS row stride (bytes)
};

template <int MT, int NB, int W, int GPS, bool DUMP>
__global__ void __launch_bounds__(W * 64)
msd_gemm_kernel(const int8_t *__restrict__ layers, const float *__restrict__ coef,
                const int32_t *__restrict__ lsum, const uint8_t *__restrict__ wp,
                const uint16_t *__restrict__ scale,
                float *__restrict__ part, uint16_t *__restrict__ y, int32_t *__restrict__ yint,
                int64_t M, int64_t Mpad, int64_t K, int64_t N, int64_t gps) {
    constexpr int NT = W * 64;
    constexpr int ROWS = MsdLds<MT>::ROWS, AROW = MsdLds<MT>::AROW;
    static_assert(GPS <= MsdLds<MT>::GPSMAX, "slice must fit in LDS");
    __shared__ __attribute__((aligned(16))) uint8_t sA[3 * ROWS * AROW];
    __shared__ __attribute__((aligned(16))) float sC[GPS * 4 * ROWS];

    const int64_t G = K / kGroup;
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, kc = lane >> 4;
    const int64_t NBLK = N / 16;
    const int64_t m0 = (int64_t)blockIdx.z * ROWS;
    const int64_t g_begin = (int64_t)blockIdx.y * gps;
    const int ng = (int)((g_begin + gps < G ? g_begin + gps : G) - g_begin);    // groups of this slice
    // N % 64 == 0 and NB divides 4: a wave's blocks are all in or all out; a
    // wave past the end runs on the last blocks and stores nothing
    const int64_t nbw = ((int64_t)blockIdx.x * W + wave) * NB;
    const bool wave_cols = nbw < NBLK;
    const int64_t nb0 = wave_cols ? nbw : NBLK - NB;

    // ---- weight tiles and scales: three register sets in a ring ----------------
    // Wave-uniform base pointers (scalar registers) plus one fixed 32-bit lane
    // offset: a group only moves the scalar base, so no per-group vector
    // address is ever formed (or kept live).
    const uint8_t *wu = wp + (nb0 * G + g_begin) * kTileBytes;
    const uint16_t *su = scale + g_begin * N + nb0 * 16;
    const uint32_t woff = (uint32_t)lane * 16u;
    u32x4_t wr[3][NB];
    uint16_t sr[3][NB];
    auto load_w = [&](int gl, u32x4_t (&wd)[NB], uint16_t (&sd)[NB]) {   // gl: group within the slice
        const int gc = __builtin_amdgcn_readfirstlane(gl < ng ? gl : ng - 1);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            wd[b] = ld128(wu + ((int64_t)b * G + gc) * kTileBytes + woff);
        if constexpr (!DUMP) {
#pragma unroll
            for (int b = 0; b < NB; ++b) sd[b] = su[(int64_t)gc * N + b * 16 + j];
        }
    };

    // ---- layers and coefficients of the slice into LDS ------------------------
    // chunk c: layer l, row, 16-byte piece p of the slice's gps*128 bytes
    {
        // every thread issues all of its layer and coefficient loads, then the
        // first two groups' weights, then stores the layers and coefficients:
        // the load counter is in order, so the stores (and the barrier) wait
        // for one round trip of the slice only, not for the weights, which
        // stay in flight into the first steps
        // every group slot of the slice is filled: slots past a short final
        // slice copy its last group (finite bytes, multiplied by zero
        // coefficients), so the chunk count and its divisions are static
        constexpr int PIECES = GPS * 8;                            // 16-byte pieces per row
        constexpr int CMAX = 3 * ROWS * PIECES;
        constexpr int CPT = (CMAX + NT - 1) / NT;
        constexpr int CN = GPS * 4 * ROWS;                         // coefficients of the slice
        constexpr int CFT = (CN + NT - 1) / NT;
        u32x4_t v[CPT];
        float cv[CFT];
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c1 = u * NT + tid, c = c1 < CMAX ? c1 : CMAX - 1;
            const int lr = c / PIECES, pc = c % PIECES;                // lr = l * ROWS + row
            const int l = lr / ROWS, row = lr % ROWS;
            const int gl = pc / 8 < ng ? pc / 8 : ng - 1;
            v[u] = ld128(layers + (l * Mpad + m0 + row) * K + (g_begin + gl) * kGroup + (pc % 8) * 16);
        }
#pragma unroll
        for (int u = 0; u < CFT; ++u) {
            const int i1 = u * NT + tid, i = i1 < CN ? i1 : CN - 1;
            const int gl = i / (4 * ROWS), lr = i % (4 * ROWS);
            const int gc = gl < ng ? gl : ng - 1;                  // in bounds; zeroed below
            cv[u] = coef[((g_begin + gc) * 4 + lr / ROWS) * Mpad + m0 + lr % ROWS];
        }
        load_w(0, wr[0], sr[0]);
        load_w(1, wr[1], sr[1]);
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = u * NT + tid;
            if (CMAX % NT == 0 || c < CMAX) {
                const int lr = c / PIECES, pc = c % PIECES;
                *reinterpret_cast<u32x4_t *>(&sA[lr * AROW + pc * 16]) = v[u];
            }
        }
#pragma unroll
        for (int u = 0; u < CFT; ++u) {
            const int i = u * NT + tid;
            if (CN % NT == 0 || i < CN) sC[i] = i / (4 * ROWS) < ng ? cv[u] : 0.f;
        }
    }
    __syncthreads();

    float yacc[NB][MT][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[b][mt][r] = 0.f;

    auto step = [&](int gl, const u32x4_t (&wc)[NB], const uint16_t (&sc)[NB], u32x4_t (&wn)[NB],
                    uint16_t (&sn)[NB]) {
        // keep each group's code in its own scheduling region: hoisting the
        // next groups' LDS reads would only raise register pressure
        __builtin_amdgcn_sched_barrier(0);
        load_w(gl + 2, wn, sn);
        u32x4_t bop[NB][2];
        float s[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            bop[b][0] = weight_u4(wc[b][0], wc[b][1]);
            bop[b][1] = weight_u4(wc[b][2], wc[b][3]);
            s[b] = DUMP ? 0.f : h2f<DT_F16>(sc[b]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            u32x4_t a[3][2];
            float c[4][4];
#pragma unroll
            for (int l = 0; l < 3; ++l) {
                const uint8_t *ap = sA + (l * ROWS + mt * 16 + j) * AROW + gl * kGroup + 32 * kc;
                a[l][0] = *reinterpret_cast<const u32x4_t *>(ap);
                a[l][1] = *reinterpret_cast<const u32x4_t *>(ap + 16);
            }
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const f32x4_t cv = *reinterpret_cast<const f32x4_t *>(&sC[(gl * 4 + l) * ROWS + mt * 16 + 4 * kc]);
#pragma unroll
                for (int r = 0; r < 4; ++r) c[l][r] = cv[r];
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                i32x4_t Y[3];
#pragma unroll
                for (int l = 0; l < 3; ++l) {
                    Y[l] = mfma_i8_16x16x64(a[l][0], bop[b][0], i32x4_t{0, 0, 0, 0});
                    Y[l] = mfma_i8_16x16x64(a[l][1], bop[b][1], Y[l]);
                }
                if constexpr (DUMP) {
                    if (wave_cols) {
#pragma unroll
                        for (int l = 0; l < 3; ++l)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int64_t row = m0 + 16 * mt + 4 * kc + r;
                                if (row < M && gl < ng)
                                    yint[(((g_begin + gl) * 3 + l) * M + row) * N + (nb0 + b) * 16 + j] =
                                        Y[l][r] - 8 * lsum[((g_begin + gl) * 3 + l) * Mpad + row];
                            }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float t = __builtin_fmaf((float)Y[0][r], c[0][r], -c[3][r]);
                        t = __builtin_fmaf((float)Y[1][r], c[1][r], t);
                        t = __builtin_fmaf((float)Y[2][r], c[2][r], t);
                        yacc[b][mt][r] += s[b] * t;
                    }
                }
            }
        }
        // the accumulators are consumed only by the final (conditional)
        // stores; without this tie the compiler sinks every group's merge to
        // those stores and keeps all products and coefficients live
        if constexpr (!DUMP) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(yacc[b][mt][r]));
        }
    };
    // fully unrolled: the ring index of every register set is static and the
    // counters of outstanding loads stay exact (steps past a short final slice
    // multiply zero coefficients)
#pragma unroll
    for (int gl = 0; gl < GPS; ++gl) {
        if (gl % 3 == 0) step(gl, wr[0], sr[0], wr[2], sr[2]);
        if (gl % 3 == 1) step(gl, wr[1], sr[1], wr[0], sr[0]);
        if (gl % 3 == 2) step(gl, wr[2], sr[2], wr[1], sr[1]);
    }

    if constexpr (DUMP) return;
    if (!wave_cols) return;
    if (gridDim.y > 1) {
        // K slices: fp32 partial sums in the matrix-core result layout, one
        // contiguous 16-byte store per lane and tile (padding rows included;
        // their layers are zero)
        float *ps = part + (((int64_t)blockIdx.y * gridDim.z + blockIdx.z) * NBLK + nb0) * (MT * 256);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<f32x4_t *>(ps + (b * MT + mt) * 256 + lane * 4) =
                    f32x4_t{yacc[b][mt][0], yacc[b][mt][1], yacc[b][mt][2], yacc[b][mt][3]};
        return;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * mt + 4 * kc + r;
                const int64_t col = (nb0 + b) * 16 + j;
                if (row < M) y[row * N + col] = f2h<DT_F16>(yacc[b][mt][r]);
            }
}

// One-row MSD (M = 1, the shape of the page's worked example, §4.3): the
// decomposition, the integer products and the merge in one launch.  A
// workgroup owns NB 16-column blocks; its 16 waves split K (wave w takes the
// groups [w*SG, (w+1)*SG)) and add their sums through LDS at the end, in wave
// order, so no partial sums reach memory and no other launch is needed.  For
// each of its groups a wave decomposes the row's 128 values itself (two per
// lane, the fp32 steps of msd_decompose_kernel; A_max and the layer sums by
// wave reductions), writes the layer bytes to its own LDS row in the order
// the matrix-core operand takes (byte p of each 8-value chunk holds value
// perm8(p)) and every lane reads its k-block of that row, so all 16 result
// rows equal row 0 and no lane is masked.  The next group's weight tiles,
// scales and x values are requested before the current group is used (two
// register sets).  DUMP writes the per-group integer products Y_j - 8 S_j
// ([G][3][1][N], as the product kernel's test hook) instead of y.
template <int NB, bool DUMP>
__global__ void __launch_bounds__(1024)
msd_row_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
               uint16_t *__restrict__ y, int32_t *__restrict__ yint, int64_t K, int64_t N) {
    constexpr int NW = 16;
    __shared__ __attribute__((aligned(16))) uint8_t sL[NW][3][kGroup];
    __shared__ float red[NW][NB * 16];
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, kc = lane >> 4;
    const int64_t G = K / kGroup;
    const int64_t SG = (G + NW - 1) / NW;
    const int64_t gb = (int64_t)wave * SG;
    const int ns = (int)(gb < G ? (gb + SG < G ? SG : G - gb) : 0);     // this wave's groups
    const int64_t nb0 = (int64_t)blockIdx.x * NB;
    const uint8_t *wu = wp + nb0 * G * kTileBytes;                      // tile (b, g) at (b*G + g) KB
    const uint32_t woff = (uint32_t)lane * 16u;

    // group gl of the slice (clamped to the slice's last; a wave without
    // groups reads group 0 and uses nothing): every load is unconditional
    auto load = [&](int gl, u32x4_t (&wd)[NB], uint16_t (&sd)[NB], uint32_t &xd) {
        const int64_t g = ns > 0 ? gb + (gl < ns ? gl : ns - 1) : 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) wd[b] = ld128(wu + ((int64_t)b * G + g) * kTileBytes + woff);
        if constexpr (!DUMP) {
#pragma unroll
            for (int b = 0; b < NB; ++b) sd[b] = scale[g * N + (nb0 + b) * 16 + j];
        }
        xd = *reinterpret_cast<const uint32_t *>(x + g * kGroup + 2 * lane);
    };
    // byte positions of this lane's two values (2*lane, 2*lane + 1) in the
    // operand order of their 8-value chunk
    const int q0 = 2 * (lane & 3);
    const int pos0 = (lane >> 2) * 8 + (q0 < 4 ? 2 * q0 : 2 * (q0 - 4) + 1);
    const int pos1 = (lane >> 2) * 8 + (q0 + 1 < 4 ? 2 * (q0 + 1) : 2 * (q0 + 1 - 4) + 1);

    float yacc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) yacc[b] = 0.f;

    auto step = [&](int gl, const u32x4_t (&wc)[NB], const uint16_t (&sc)[NB], uint32_t xc, u32x4_t (&wn)[NB],
                    uint16_t (&sn)[NB], uint32_t &xn) {
        load(gl + 1, wn, sn, xn);
        const int64_t g = gb + gl;
        // eq.1-7 for the row's group g
        const float a0 = h2f<DT_F16>((uint16_t)(xc & 0xFFFFu)), a1 = h2f<DT_F16>((uint16_t)(xc >> 16));
        const float am = wave_max_nonneg(fmaxf(fabsf(a0), fabsf(a1)));
        int l0[3], l1[3], ls[3];
        msd_decompose(a0, am, l0[0], l0[1], l0[2]);
        msd_decompose(a1, am, l1[0], l1[1], l1[2]);
#pragma unroll
        for (int q = 0; q < 3; ++q) ls[q] = wave_sum_i32(l0[q] + l1[q]);   // exact in int32
        const float c0 = am * kR0, c1 = am * kR1, c2 = am * kR2;
        const float c3 = 8.f * __builtin_fmaf(c0, (float)ls[0], __builtin_fmaf(c1, (float)ls[1], c2 * (float)ls[2]));
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            sL[wave][q][pos0] = (uint8_t)(int8_t)l0[q];
            sL[wave][q][pos1] = (uint8_t)(int8_t)l1[q];
        }
        // one wave's LDS accesses complete in order: the reads below see the
        // writes above, and the next group's writes follow these reads
        __builtin_amdgcn_wave_barrier();
        u32x4_t a[3][2];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            a[q][0] = *reinterpret_cast<const u32x4_t *>(&sL[wave][q][32 * kc]);
            a[q][1] = *reinterpret_cast<const u32x4_t *>(&sL[wave][q][32 * kc + 16]);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4_t b0 = weight_u4(wc[b][0], wc[b][1]), b1 = weight_u4(wc[b][2], wc[b][3]);
            i32x4_t Y[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                Y[q] = mfma_i8_16x16x64(a[q][0], b0, i32x4_t{0, 0, 0, 0});
                Y[q] = mfma_i8_16x16x64(a[q][1], b1, Y[q]);
            }
            if constexpr (DUMP) {
                if (kc == 0) {
#pragma unroll
                    for (int q = 0; q < 3; ++q) yint[(g * 3 + q) * N + (nb0 + b) * 16 + j] = Y[q][0] - 8 * ls[q];
                }
            } else {
                float t = __builtin_fmaf((float)Y[0][0], c0, -c3);
                t = __builtin_fmaf((float)Y[1][0], c1, t);
                t = __builtin_fmaf((float)Y[2][0], c2, t);
                yacc[b] += h2f<DT_F16>(sc[b]) * t;
            }
        }
    };

    u32x4_t wr0[NB], wr1[NB];
    uint16_t sr0[NB], sr1[NB];
    uint32_t xr0, xr1;
    load(0, wr0, sr0, xr0);
    int gl = 0;
    for (; gl + 1 < ns; gl += 2) {
        step(gl, wr0, sr0, xr0, wr1, sr1, xr1);
        step(gl + 1, wr1, sr1, xr1, wr0, sr0, xr0);
    }
    if (gl < ns) step(gl, wr0, sr0, xr0, wr1, sr1, xr1);

    if constexpr (DUMP) return;
    if (kc == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) red[wave][b * 16 + j] = yacc[b];
    }
    __syncthreads();
    if (tid < NB * 16) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w][tid];
        y[nb0 * 16 + tid] = f2h<DT_F16>(sum);
    }
}

// Sum of the K slices' partial sums (matrix-core result layout: per row chunk z,
// 16-column block nb and 16-row tile mt, 64 lanes x 4 result registers) and
// rounding to fp16.  One thread per lane and tile; slice stride `slice` floats.
// The slices of up to eight k are loaded before any is added (one memory
// round trip per eight slices); the sum keeps the order 0 .. ksplit-1.
__global__ void __launch_bounds__(256)
msd_reduce_kernel(const float *__restrict__ part, uint16_t *__restrict__ y, int64_t M, int64_t N, int mt_count,
                  int64_t nlanes, int64_t slice, int ksplit) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;      // (z, nb, mt, lane)
    if (t >= nlanes) return;
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(part + t * 4);
    for (int k0 = 1; k0 < ksplit; k0 += 8) {
        f32x4_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + i < ksplit ? k0 + i : ksplit - 1;   // in bounds; not added past ksplit
            v[i] = *reinterpret_cast<const f32x4_t *>(part + k * slice + t * 4);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (k0 + i < ksplit) acc += v[i];
    }
    const int lane = (int)(t & 63);
    const int64_t tile = t >> 6;
    const int mt = (int)(tile % mt_count);
    const int64_t nb = (tile / mt_count) % (N / 16);
    const int64_t z = tile / mt_count / (N / 16);
    const int64_t row0 = (z * mt_count + mt) * 16 + 4 * (lane >> 4);
    const int64_t col = nb * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (row0 + r < M) y[(row0 + r) * N + col] = f2h<DT_F16>(acc[r]);
}

// Basic pipeline (the MSD page's §6.1 stage order with the integer products
// passed through memory, for comparison with the fused kernel): merge of the
// per-group products Y_j [G][3][M][N] (signed, eq.9) read back from memory,
//   y[m][n] = RNE( sum_g s[g][n] * (Y_1 c_1 + Y_2 c_2 + Y_3 c_3) ),
// c_j = A_max / (7.49 * 14.98^(j-1)) from the decomposition (eqs.10-11), in
// fp32; 4 columns per lane.
__global__ void __launch_bounds__(256)
msd_merge_kernel(const int32_t *__restrict__ yint, const float *__restrict__ coef,
                 const uint16_t *__restrict__ scale, uint16_t *__restrict__ y, int64_t M, int64_t Mpad,
                 int64_t N, int64_t G) {
    const int64_t nv = N / 4;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < M * nv; idx += (int64_t)gridDim.x * 256) {
        const int64_t m = idx / nv, c0 = (idx % nv) * 4;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int64_t g = 0; g < G; ++g) {
            const float k0 = coef[(g * 4 + 0) * Mpad + m], k1 = coef[(g * 4 + 1) * Mpad + m],
                        k2 = coef[(g * 4 + 2) * Mpad + m];
            const i32x4_t y0 = *reinterpret_cast<const i32x4_t *>(yint + ((g * 3 + 0) * M + m) * N + c0);
            const i32x4_t y1 = *reinterpret_cast<const i32x4_t *>(yint + ((g * 3 + 1) * M + m) * N + c0);
            const i32x4_t y2 = *reinterpret_cast<const i32x4_t *>(yint + ((g * 3 + 2) * M + m) * N + c0);
            const uint2 sv = *reinterpret_cast<const uint2 *>(scale + g * N + c0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float t = (float)y0[j] * k0;
                t = __builtin_fmaf((float)y1[j], k1, t);
                t = __builtin_fmaf((float)y2[j], k2, t);
                const uint32_t sw = j < 2 ? sv.x : sv.y;
                acc[j] = __builtin_fmaf(h2f<DT_F16>((uint16_t)(sw >> (16 * (j & 1)))), t, acc[j]);
            }
        }
        uint2 out;
        out.x = (uint32_t)f2h<DT_F16>(acc[0]) | (uint32_t)f2h<DT_F16>(acc[1]) << 16;
        out.y = (uint32_t)f2h<DT_F16>(acc[2]) | (uint32_t)f2h<DT_F16>(acc[3]) << 16;
        *reinterpret_cast<uint2 *>(y + m * N + c0) = out;
    }
}

// Plain-order copy of the layers for the test hook.
__global__ void msd_layers_plain_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst, int64_t M,
                                        int64_t Mpad, int64_t K) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 3 * M * K) return;
    const int64_t l = idx / (M * K), m = (idx / K) % M, k = idx % K;
    const int64_t base = k & ~7LL;
    int p = 0;
    while (perm8(p) != (int)(k & 7)) ++p;
    dst[idx] = src[(l * Mpad + m) * K + base + p];
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Configurations of msd_gemm_kernel: (16-row tiles per workgroup, column
// blocks per wave, waves).  Index 0 is the default; the others are kept for
// tuning through the test hook.
struct MsdCfg { int mt, nb, waves; };
static constexpr MsdCfg kMsdCfgs[] = {{2, 4, 8}, {2, 4, 4}, {1, 4, 8}, {4, 2, 8}, {2, 2, 8}, {4, 4, 4}};
static std::atomic<int> g_msd_cfg{-1};       // -1: automatic
int msd_config_count() { return (int)(sizeof(kMsdCfgs) / sizeof(kMsdCfgs[0])); }
void set_msd_config(int idx) { g_msd_cfg.store(idx, std::memory_order_relaxed); }

static MsdPlan msd_plan_cfg(int64_t M, int64_t K, int64_t N, const MsdCfg &c) {
    MsdPlan p{};
    const int64_t G = K / kGroup;
    p.mt = c.mt;
    while (p.mt > 1 && 16 * (p.mt / 2) >= M) p.mt /= 2;      // no more row tiles than rows
    p.mchunks = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
    if (p.mchunks < 1) p.mchunks = 1;
    p.mpad = (M + 63) / 64 * 64;                               // layers padded for every configuration
    if (p.mpad < 64) p.mpad = 64;
    p.nb = c.nb;
    p.waves = c.waves;
    const int64_t colwg = (N / 16 + p.nb * p.waves - 1) / (p.nb * p.waves);
    // slice length: the longest power of two that fits in LDS and still
    // gives the grid about 2048 waves (else the shortest, 2 groups)
    const int64_t gpsmax = p.mt == 1 ? MsdLds<1>::GPSMAX : p.mt == 2 ? MsdLds<2>::GPSMAX : MsdLds<4>::GPSMAX;
    const int64_t target = 2048 / p.waves;
    p.gps = 2;
    for (int64_t g = gpsmax; g >= 2; g /= 2)
        if (colwg * p.mchunks * ((G + g - 1) / g) >= target || g == 2) { p.gps = g; break; }
    p.ksplit = (int)((G + p.gps - 1) / p.gps);
    p.off_coef = 0;
    p.off_lsum = align_up(p.off_coef + sizeof(float) * (size_t)(G * 4 * p.mpad), 256);
    p.off_amax = align_up(p.off_lsum + sizeof(int32_t) * (size_t)(G * 3 * p.mpad), 256);
    p.off_layers = align_up(p.off_amax + sizeof(float) * (size_t)(M * G), 256);
    p.off_part = align_up(p.off_layers + (size_t)(3 * p.mpad * K), 256);
    const int64_t rows_cov = (int64_t)p.mchunks * 16 * p.mt;   // rows covered by the row chunks
    p.total = align_up(p.off_part + (p.ksplit > 1 ? sizeof(float) * (size_t)(p.ksplit * rows_cov * N) : 0), 256);
    return p;
}

MsdPlan msd_plan(int64_t M, int64_t K, int64_t N) {
    int idx = g_msd_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= msd_config_count()) idx = 0;
    return msd_plan_cfg(M, K, N, kMsdCfgs[idx]);
}

size_t msd_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    // the largest plan over all configurations, so that a size queried once
    // fits whichever configuration runs
    size_t mx = 0;
    for (int i = 0; i < msd_config_count(); ++i) {
        const size_t t = msd_plan_cfg(M, K, N, kMsdCfgs[i]).total;
        mx = t > mx ? t : mx;
    }
    return mx;
}

template <bool DUMP>
static hipError_t msd_gemm_launch(const MsdPlan &p, const int8_t *layers, const float *coef,
                                  const int32_t *lsum, const void *wp,
                                  const void *scale, float *part, void *y, int32_t *yint, int64_t M,
                                  int64_t K, int64_t N, int ksplit, int64_t gps, hipStream_t stream) {
    const int64_t colwg = (N / 16 + p.nb * p.waves - 1) / (p.nb * p.waves);
    const dim3 grid((unsigned)colwg, (unsigned)ksplit, (unsigned)p.mchunks);
    const dim3 block(p.waves * 64);
#define W4_MSD_LAUNCH(MTV, NBV, WV, GV)                                                                       \
    if (p.mt == MTV && p.nb == NBV && p.waves == WV && gps == GV) {                                            \
        hipLaunchKernelGGL((msd_gemm_kernel<MTV, NBV, WV, GV, DUMP>), grid, block, 0, stream, layers, coef,      \
                           lsum, (const uint8_t *)wp, (const uint16_t *)scale, part, (uint16_t *)y, yint, M, p.mpad, \
                           K, N, gps);                                                                         \
        return hipGetLastError();                                                                              \
    }
#define W4_MSD_GPS1(MTV, NBV, WV) W4_MSD_LAUNCH(MTV, NBV, WV, 2) W4_MSD_LAUNCH(MTV, NBV, WV, 4)               \
    W4_MSD_LAUNCH(MTV, NBV, WV, 8) W4_MSD_LAUNCH(MTV, NBV, WV, 16)
#define W4_MSD_GPS2(MTV, NBV, WV) W4_MSD_LAUNCH(MTV, NBV, WV, 2) W4_MSD_LAUNCH(MTV, NBV, WV, 4)               \
    W4_MSD_LAUNCH(MTV, NBV, WV, 8)
#define W4_MSD_GPS4(MTV, NBV, WV) W4_MSD_LAUNCH(MTV, NBV, WV, 2) W4_MSD_LAUNCH(MTV, NBV, WV, 4)
    W4_MSD_GPS2(2, 4, 8) W4_MSD_GPS2(2, 4, 4) W4_MSD_GPS1(1, 4, 8) W4_MSD_GPS4(4, 2, 8)
    W4_MSD_GPS2(2, 2, 8) W4_MSD_GPS4(4, 4, 4)
    // configurations reduced to fewer row tiles for small M
    W4_MSD_GPS1(1, 4, 4) W4_MSD_GPS1(1, 2, 8)
#undef W4_MSD_GPS1
#undef W4_MSD_GPS2
#undef W4_MSD_GPS4
#undef W4_MSD_LAUNCH
    return hipErrorInvalidValue;
}

static hipError_t msd_pre(const MsdPlan &p, const void *x, uint8_t *ws, int64_t M, int64_t K,
                          hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t pairs = p.mpad * G;
    hipLaunchKernelGGL(msd_decompose_kernel, dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, stream,
                       (const uint16_t *)x, (float *)(ws + p.off_coef), (int32_t *)(ws + p.off_lsum),
                       (float *)(ws + p.off_amax),
                       (int8_t *)(ws + p.off_layers), M, p.mpad, K);
    return hipGetLastError();
}

static hipError_t launch_msd_plan(const MsdPlan &p, const void *x, const void *wp, const void *scale, void *y,
                                  int64_t M, int64_t K, int64_t N, void *workspace, hipStream_t stream) {
    uint8_t *ws = (uint8_t *)workspace;
    hipError_t err = msd_pre(p, x, ws, M, K, stream);
    if (err != hipSuccess) return err;
    err = msd_gemm_launch<false>(p, (const int8_t *)(ws + p.off_layers), (const float *)(ws + p.off_coef),
                                 (const int32_t *)(ws + p.off_lsum), wp,
                                 scale, (float *)(ws + p.off_part), y, nullptr, M, K, N, p.ksplit, p.gps, stream);
    if (err != hipSuccess || p.ksplit == 1) return err;
    const int64_t slice = (int64_t)p.mchunks * 16 * p.mt * N;     // floats per K slice
    const int64_t nlanes = slice / 4;
    hipLaunchKernelGGL(msd_reduce_kernel, dim3((unsigned)((nlanes + 255) / 256)), dim3(256), 0, stream,
                       (const float *)(ws + p.off_part), (uint16_t *)y, M, N, p.mt, nlanes, slice, p.ksplit);
    return hipGetLastError();
}

// One row: the one-launch kernel above (N % 64 == 0 by contract, so the
// grid covers the columns exactly); needs no workspace.
constexpr int kMsdRowNb = 4;
template <bool DUMP>
static hipError_t launch_msd_row(const void *x, const void *wp, const void *scale, void *y, int32_t *yint,
                                 int64_t K, int64_t N, hipStream_t stream) {
    hipLaunchKernelGGL((msd_row_kernel<kMsdRowNb, DUMP>), dim3((unsigned)(N / (16 * kMsdRowNb))), dim3(1024), 0,
                       stream, (const uint16_t *)x, (const uint8_t *)wp, (const uint16_t *)scale, (uint16_t *)y,
                       yint, K, N);
    return hipGetLastError();
}

hipError_t launch_msd(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                      int64_t N, void *workspace, hipStream_t stream) {
    if (M == 1) return launch_msd_row<false>(x, wp, scale, y, nullptr, K, N, stream);
    return launch_msd_plan(msd_plan(M, K, N), x, wp, scale, y, M, K, N, workspace, stream);
}


// ---- the MSD call without a caller workspace ---------------------------------
// For callers that cannot allocate device memory: the workspace lives in a
// file-scope device array of kMsdScratchBytes that every GPU the library runs
// on holds until the process ends.  In host code `scratch` is only a host-side
// stand-in for that array; its device address is taken once per device, with
// that device current, through hipGetSymbolAddress, and only that address is
// ever handed to kernels.  Nothing in the workspace needs to start at zero
// (every byte a kernel reads was written earlier in the same call), so no
// clearing is done.  All calls on one GPU share the array: calls that overlap
// in time on one GPU (different streams without ordering) race.
static __device__ __align__(256) uint8_t scratch[kMsdScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kScratchDevices];
}  // namespace

static hipError_t msd_scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    ScratchSlot &sl = g_scratch[dev];
    std::call_once(sl.once, [&] { sl.err = hipGetSymbolAddress(&sl.ptr, HIP_SYMBOL(scratch)); });
    if (sl.err != hipSuccess) return sl.err;
    if (!sl.ptr) return hipErrorInvalidSymbol;
    *out = sl.ptr;
    return hipSuccess;
}

size_t msd_noalloc_bytes(int64_t M, int64_t K, int64_t N) { return M == 1 ? 0 : msd_plan(M, K, N).total; }

hipError_t launch_msd_noalloc(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                              int64_t N, hipStream_t stream) {
    if (M == 1) return launch_msd_row<false>(x, wp, scale, y, nullptr, K, N, stream);     // no workspace
    const MsdPlan p = msd_plan(M, K, N);     // the plan that runs: its own workspace size is checked
    if (p.total > kMsdScratchBytes) return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = msd_scratch_ptr(&ws);
    if (e != hipSuccess) return e;
    return launch_msd_plan(p, x, wp, scale, y, M, K, N, ws, stream);
}

size_t msd_basic_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    return align_up(msd_workspace_bytes(M, K, N), 256) + sizeof(int32_t) * (size_t)(K / kGroup) * 3 * (size_t)M * (size_t)N;
}

hipError_t launch_msd_basic(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                            int64_t N, void *workspace, hipStream_t stream) {
    const MsdPlan p = msd_plan(M, K, N);
    uint8_t *ws = (uint8_t *)workspace;
    int32_t *yint = (int32_t *)(ws + align_up(msd_workspace_bytes(M, K, N), 256));
    hipError_t err = msd_pre(p, x, ws, M, K, stream);
    if (err != hipSuccess) return err;
    err = msd_gemm_launch<true>(p, (const int8_t *)(ws + p.off_layers), (const float *)(ws + p.off_coef),
                                (const int32_t *)(ws + p.off_lsum), wp, nullptr, nullptr, nullptr, yint, M, K, N,
                                p.ksplit, p.gps, stream);
    if (err != hipSuccess) return err;
    int64_t blocks = (M * (N / 4) + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(msd_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, yint,
                       (const float *)(ws + p.off_coef), (const uint16_t *)scale, (uint16_t *)y, M, p.mpad, N,
                       K / kGroup);
    return hipGetLastError();
}

hipError_t launch_msd_intermediates(const void *x, const void *wp, int64_t M, int64_t K, int64_t N,
                                    float *amax, int8_t *layers, int32_t *yint, void *workspace,
                                    hipStream_t stream) {
    const MsdPlan p = msd_plan(M, K, N);
    uint8_t *ws = (uint8_t *)workspace;
    hipError_t err = msd_pre(p, x, ws, M, K, stream);
    if (err != hipSuccess) return err;
    err = hipMemcpyAsync(amax, ws + p.off_amax, sizeof(float) * (size_t)(M * (K / kGroup)),
                         hipMemcpyDeviceToDevice, stream);
    if (err != hipSuccess) return err;
    const int64_t n = 3 * M * K;
    hipLaunchKernelGGL(msd_layers_plain_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const int8_t *)(ws + p.off_layers), layers, M, p.mpad, K);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the products of every group are written separately (one row: by the
    // one-launch kernel, from its own decomposition)
    if (M == 1) return launch_msd_row<true>(x, wp, nullptr, nullptr, yint, K, N, stream);
    return msd_gemm_launch<true>(p, (const int8_t *)(ws + p.off_layers), (const float *)(ws + p.off_coef),
                                 (const int32_t *)(ws + p.off_lsum), wp,
                                 nullptr, nullptr, nullptr, yint, M, K, N, p.ksplit, p.gps, stream);
}

}  // namespace w4
