// fzero.hip — floating-point zero points for the dense integer-weight GEMMs
// (the Humming article's descriptor lists zero points among the quantization
// parameters; here they are values of the activation dtype).
//
// dequant(W)[k][n] = (u[k][n] - zf[g][n]) * s[g][n] with u the unsigned code.
// An unsigned code u is stored exactly like the signed value q = u - off
// (off = 8 for 4-bit, 128 for 8-bit weights), so the signed GEMM path already
// computes sum_k x * (u - off) * s; the rest,
//   C[m][n] = sum_g S[m][g] * (zf[g][n] - off) * s[g][n],
//   S[m][g] = sum over the rows k of scale group g of x[m][k],
// is formed here in fp32 and subtracted by the GEMM epilogue before the
// secondary scale and the one rounding.
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

// S[m][g]: one 256-thread workgroup per row; eight elements per lane per
// 128-bit load, partial sums added per scale group in LDS.
template <int DT>
__global__ void __launch_bounds__(256) fz_rowsum_kernel(const uint16_t *__restrict__ x, float *__restrict__ S,
                                                        int64_t K, int64_t gs) {
    extern __shared__ float sg[];
    const int64_t m = blockIdx.x;
    const int64_t G = K / gs;
    for (int64_t g = threadIdx.x; g < G; g += 256) sg[g] = 0.f;
    __syncthreads();
    for (int64_t c = threadIdx.x; c < K / 8; c += 256) {
        const u32x4_t v = ld128(x + m * K + c * 8);
        float p = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) p += h2f<DT>((uint16_t)(v[t] & 0xFFFFu)) + h2f<DT>((uint16_t)(v[t] >> 16));
        atomicAdd(&sg[c * 8 / gs], p);
    }
    __syncthreads();
    for (int64_t g = threadIdx.x; g < G; g += 256) S[m * G + g] = sg[g];
}

// C[m][n] for 16 rows per workgroup row and one column per lane.
template <int DT>
__global__ void __launch_bounds__(256) fz_corr_kernel(const float *__restrict__ S, const uint16_t *__restrict__ scale,
                                                      const uint16_t *__restrict__ zf, float *__restrict__ C,
                                                      int64_t M, int64_t N, int64_t G, float off) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    if (n >= N) return;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int64_t g = 0; g < G; ++g) {
        const float zs = (h2f<DT>(zf[g * N + n]) - off) * h2f<DT>(scale[g * N + n]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t m = m0 + i < M ? m0 + i : M - 1;
            acc[i] = __builtin_fmaf(S[m * G + g], zs, acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (m0 + i < M) C[(m0 + i) * N + n] = acc[i];
}

size_t fzero_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t gs) {
    const size_t s_bytes = ((size_t)M * (size_t)(K / gs) * sizeof(float) + 255) & ~(size_t)255;
    return s_bytes + (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_fzero_corr(const void *x, const void *scale, const void *zf, int64_t M, int64_t K, int64_t N,
                             int64_t gs, int bits, int dt, void *workspace, float **corr, hipStream_t stream) {
    const int64_t G = K / gs;
    float *S = (float *)workspace;
    float *C = (float *)((uint8_t *)workspace + (((size_t)M * (size_t)G * sizeof(float) + 255) & ~(size_t)255));
    *corr = C;
    const float off = bits == 8 ? 128.f : 8.f;
    const size_t lds = (size_t)G * sizeof(float);
    const dim3 cgrid((unsigned)((N + 255) / 256), (unsigned)((M + 15) / 16));
    if (dt == DT_BF16) {
        hipLaunchKernelGGL(fz_rowsum_kernel<DT_BF16>, dim3((unsigned)M), dim3(256), lds, stream,
                           (const uint16_t *)x, S, K, gs);
        hipLaunchKernelGGL(fz_corr_kernel<DT_BF16>, cgrid, dim3(256), 0, stream, (const float *)S,
                           (const uint16_t *)scale, (const uint16_t *)zf, C, M, N, G, off);
    } else {
        hipLaunchKernelGGL(fz_rowsum_kernel<DT_F16>, dim3((unsigned)M), dim3(256), lds, stream,
                           (const uint16_t *)x, S, K, gs);
        hipLaunchKernelGGL(fz_corr_kernel<DT_F16>, cgrid, dim3(256), 0, stream, (const float *)S,
                           (const uint16_t *)scale, (const uint16_t *)zf, C, M, N, G, off);
    }
    return hipGetLastError();
}

}  // namespace w4
