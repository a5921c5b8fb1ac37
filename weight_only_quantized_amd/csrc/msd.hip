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
// Workspace (caller-owned): coef [G][3][Mpad] fp32 (A_max / (7.49*14.98^j)),
// amax [M][G] fp32, layers [3][Mpad][K] int8 in operand order, and for K
// splits > 1 partial sums [ksplit][M][N] fp32.
//
// Layer storage order: inside each aligned 8-k block, byte p holds
// k = base + {0,4,1,5,2,6,3,7}[p].  That is the order in which the int8
// operand of the weights comes out of one prepacked word
// (word & 0x0F0F0F0F gives rows 0,4,1,5; (word >> 4) & 0x0F0F0F0F gives
// 2,6,3,7), so both operands of v_mfma_i32_16x16x64_i8 see the same k in the
// same byte.
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

// One 256-thread workgroup handles 16 (row, group) pairs; 16 lanes per pair,
// 8 elements per lane.
__global__ void __launch_bounds__(256)
msd_decompose_kernel(const uint16_t *__restrict__ x, float *__restrict__ coef, float *__restrict__ amax_out,
                     int8_t *__restrict__ layers, int64_t M, int64_t Mpad, int64_t K) {
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
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    am = fmaxf(am, __shfl_xor(am, 8));          // eq.1: A_max of the (row, group)
    if (!valid) return;

    int l[3][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) msd_decompose(a[i], am, l[0][i], l[1][i], l[2][i]);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        uint64_t packed = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p) packed |= (uint64_t)(uint8_t)(int8_t)l[j][perm8(p)] << (8 * p);
        *reinterpret_cast<uint64_t *>(layers + (j * Mpad + m) * K + g * kGroup + sub * 8) = packed;
    }
    if (sub == 0) {
        coef[(g * 3 + 0) * Mpad + m] = am * kR0;
        coef[(g * 3 + 1) * Mpad + m] = am * kR1;
        coef[(g * 3 + 2) * Mpad + m] = am * kR2;
        if (real) amax_out[m * G + g] = am;
    }
}

// Signed int8 operand of one 16x16x64 step from two prepacked words.
__device__ __forceinline__ u32x4_t weight_i8(uint32_t w0, uint32_t w1) {
    return u32x4_t{codes_to_s8(w0 & 0x0F0F0F0Fu), codes_to_s8((w0 >> 4) & 0x0F0F0F0Fu),
                   codes_to_s8(w1 & 0x0F0F0F0Fu), codes_to_s8((w1 >> 4) & 0x0F0F0F0Fu)};
}

// Integer products of the three layers with the weights (eq.9) and the merge
// (eqs.10-11).  Waves split the columns (NB 16-column blocks each); a
// workgroup owns W*NB blocks, MT 16-row tiles of x rows and one K slice
// (blockIdx.y).  Lane l of v_mfma_i32_16x16x64_i8 feeds row/column l % 16,
// k-block l / 16 (32 rows of the group: prepacked chunk l / 16; step t uses its
// words 2t and 2t+1).  Result register r of lane l is row 4*(l/16) + r,
// column l % 16.
template <int MT, int NB, int W, bool DUMP>
__global__ void __launch_bounds__(W * 64)
msd_gemm_kernel(const int8_t *__restrict__ layers, const float *__restrict__ coef,
                const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
                float *__restrict__ part, uint16_t *__restrict__ y, int32_t *__restrict__ yint,
                int64_t M, int64_t Mpad, int64_t K, int64_t N, int64_t gps) {
    const int64_t G = K / kGroup;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int j = lane & 15, kc = lane >> 4;
    const int64_t nb0 = ((int64_t)blockIdx.x * W + wave) * NB;
    const int64_t ks = blockIdx.y;
    const int64_t m0 = (int64_t)blockIdx.z * 16 * MT;
    const int64_t g_begin = ks * gps;
    const int64_t g_end = g_begin + gps < G ? g_begin + gps : G;
    if (nb0 >= N / 16) return;

    float yacc[NB][MT][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[b][mt][r] = 0.f;

    for (int64_t g = g_begin; g < g_end; ++g) {
        u32x4_t bop[NB][2];
        float s[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x4_t raw = ld128(wp + ((nb0 + b) * G + g) * kTileBytes + lane * 16);
            bop[b][0] = weight_i8(raw[0], raw[1]);
            bop[b][1] = weight_i8(raw[2], raw[3]);
            s[b] = DUMP ? 0.f : h2f<DT_F16>(scale[g * N + (nb0 + b) * 16 + j]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t arow = m0 + 16 * mt + j;            // A-operand row (padded rows are zero)
            u32x4_t a[3][2];
            float c[3][4];
#pragma unroll
            for (int l = 0; l < 3; ++l) {
                const int8_t *ap = layers + (l * Mpad + arow) * K + g * kGroup + 32 * kc;
                a[l][0] = ld128(ap);
                a[l][1] = ld128(ap + 16);
                const f32x4_t cv = *reinterpret_cast<const f32x4_t *>(coef + (g * 3 + l) * Mpad + m0 + 16 * mt + 4 * kc);
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
#pragma unroll
                    for (int l = 0; l < 3; ++l)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int64_t row = m0 + 16 * mt + 4 * kc + r;
                            if (row < M) yint[((g * 3 + l) * M + row) * N + (nb0 + b) * 16 + j] = Y[l][r];
                        }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float t = (float)Y[0][r] * c[0][r] + (float)Y[1][r] * c[1][r] + (float)Y[2][r] * c[2][r];
                        yacc[b][mt][r] += s[b] * t;
                    }
                }
            }
        }
    }
    if constexpr (DUMP) return;

    const bool split = gridDim.y > 1;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * mt + 4 * kc + r;
                const int64_t col = (nb0 + b) * 16 + j;
                if (row < M) {
                    if (split) part[(ks * M + row) * N + col] = yacc[b][mt][r];
                    else y[row * N + col] = f2h<DT_F16>(yacc[b][mt][r]);
                }
            }
}

__global__ void __launch_bounds__(256)
msd_reduce_kernel(const float *__restrict__ part, uint16_t *__restrict__ y, int64_t MN, int ksplit) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;          // MN % 4 == 0 (N % 64 == 0)
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(part + i);
    for (int k = 1; k < ksplit; ++k) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(part + k * MN + i);
        acc += v;
    }
    uint32_t lo = f2h<DT_F16>(acc[0]) | ((uint32_t)f2h<DT_F16>(acc[1]) << 16);
    uint32_t hi = f2h<DT_F16>(acc[2]) | ((uint32_t)f2h<DT_F16>(acc[3]) << 16);
    *reinterpret_cast<uint2 *>(y + i) = make_uint2(lo, hi);
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

MsdPlan msd_plan(int64_t M, int64_t K, int64_t N) {
    MsdPlan p{};
    const int64_t G = K / kGroup;
    const int64_t mrows = M < 64 ? M : 64;
    p.mt = mrows <= 16 ? 1 : (mrows <= 32 ? 2 : 4);
    p.mchunks = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
    if (p.mchunks < 1) p.mchunks = 1;
    p.mpad = (int64_t)p.mchunks * 16 * p.mt;
    p.nb = 2;
    p.waves = 4;
    const int64_t colwg = N / (16 * p.nb * p.waves) + (N % (16 * p.nb * p.waves) ? 1 : 0);
    // aim for at least ~512 workgroups over K slices, each slice >= 4 groups
    int64_t ks = 1;
    while (colwg * p.mchunks * ks < 512 && G / (ks * 2) >= 4) ks *= 2;
    p.ksplit = (int)ks;
    p.gps = (G + ks - 1) / ks;
    p.off_coef = 0;
    p.off_amax = align_up(p.off_coef + sizeof(float) * (size_t)(G * 3 * p.mpad), 256);
    p.off_layers = align_up(p.off_amax + sizeof(float) * (size_t)(M * G), 256);
    p.off_part = align_up(p.off_layers + (size_t)(3 * p.mpad * K), 256);
    p.total = align_up(p.off_part + (p.ksplit > 1 ? sizeof(float) * (size_t)(p.ksplit * M * N) : 0), 256);
    return p;
}

template <bool DUMP>
static hipError_t msd_gemm_launch(const MsdPlan &p, const int8_t *layers, const float *coef, const void *wp,
                                  const void *scale, float *part, void *y, int32_t *yint, int64_t M,
                                  int64_t K, int64_t N, int ksplit, int64_t gps, hipStream_t stream) {
    const int64_t colwg = (N / 16 + p.nb * p.waves - 1) / (p.nb * p.waves);
    const dim3 grid((unsigned)colwg, (unsigned)ksplit, (unsigned)p.mchunks);
    const dim3 block(p.waves * 64);
#define W4_MSD_LAUNCH(MTV)                                                                                     \
    hipLaunchKernelGGL((msd_gemm_kernel<MTV, 2, 4, DUMP>), grid, block, 0, stream, layers, coef,                 \
                       (const uint8_t *)wp, (const uint16_t *)scale, part, (uint16_t *)y, yint, M, p.mpad, K, N, \
                       gps)
    if (p.mt == 1) W4_MSD_LAUNCH(1);
    else if (p.mt == 2) W4_MSD_LAUNCH(2);
    else W4_MSD_LAUNCH(4);
#undef W4_MSD_LAUNCH
    return hipGetLastError();
}

static hipError_t msd_pre(const MsdPlan &p, const void *x, uint8_t *ws, int64_t M, int64_t K,
                          hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t pairs = p.mpad * G;
    hipLaunchKernelGGL(msd_decompose_kernel, dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, stream,
                       (const uint16_t *)x, (float *)(ws + p.off_coef), (float *)(ws + p.off_amax),
                       (int8_t *)(ws + p.off_layers), M, p.mpad, K);
    return hipGetLastError();
}

hipError_t launch_msd(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                      int64_t N, void *workspace, hipStream_t stream) {
    const MsdPlan p = msd_plan(M, K, N);
    uint8_t *ws = (uint8_t *)workspace;
    hipError_t err = msd_pre(p, x, ws, M, K, stream);
    if (err != hipSuccess) return err;
    err = msd_gemm_launch<false>(p, (const int8_t *)(ws + p.off_layers), (const float *)(ws + p.off_coef), wp,
                                 scale, (float *)(ws + p.off_part), y, nullptr, M, K, N, p.ksplit, p.gps, stream);
    if (err != hipSuccess || p.ksplit == 1) return err;
    const int64_t MN = M * N;
    hipLaunchKernelGGL(msd_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, stream,
                       (const float *)(ws + p.off_part), (uint16_t *)y, MN, p.ksplit);
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
    // one group per K slice, so every group's products are written separately
    return msd_gemm_launch<true>(p, (const int8_t *)(ws + p.off_layers), (const float *)(ws + p.off_coef), wp,
                                 nullptr, nullptr, nullptr, yint, M, K, N, (int)(K / kGroup), 1, stream);
}

}  // namespace w4
