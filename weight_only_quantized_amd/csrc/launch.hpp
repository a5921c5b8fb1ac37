// launch.hpp — internal launchers between the C-ABI layer (api.cpp) and the
// kernels.  All pointers are device pointers; shapes were validated by the
// caller.  Each launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

// layout 0: the standard tile layout; 1: the group-aligned layout (scale
// groups of 32 or 64 rows; see prepack.hip)
hipError_t launch_prepack(const void *w, void *out, int64_t E, int64_t K, int64_t N, int is_signed,
                          hipStream_t stream, int layout = 0);
hipError_t launch_unpack(const void *in, void *w, int64_t E, int64_t K, int64_t N, int is_signed,
                         hipStream_t stream, int layout = 0);

// Small-M split-K kernel (M <= 16, K <= small_max_k()).
int small_config_count();
void set_small_config(int idx);
int64_t small_max_k();
// Its two-tile form for M > 16 (K <= small2_max_k(); 32-row groups on the grid).
int64_t small2_max_k();
// gm: 128-row groups per scale group (scale and zero have K/(128*gm) rows).
// cs: optional per-column fp32 secondary scale applied before the rounding;
// cz: optional fp32 [M][N] subtracted before it (floating-point zero points).
hipError_t launch_gemm_small(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                             int64_t M, int64_t K, int64_t N, int dt, hipStream_t stream, int gm = 1,
                             const float *cs = nullptr, const float *cz = nullptr);

// Scale groups of 32 or 64 rows (weights prepacked in the group-aligned
// layout): M <= 16 and K <= small_gs_max_k().
int64_t small_gs_max_k();
hipError_t launch_gemm_small_gs(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                                int64_t M, int64_t K, int64_t N, int dt, int group_size, hipStream_t stream,
                                const float *cs = nullptr, const float *cz = nullptr);

// LDS-staged tile kernel; grouped when offsets != nullptr (then M = R rows).
// With row_src, row r of the product reads x row row_src[r] (gathered load).
int tile_config_count();
void set_tile_config(int idx);
int set_tile_halves(int enable);     // returns the previous setting
hipError_t launch_gemm_tile(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                            const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E,
                            int dt, hipStream_t stream, const int32_t *row_src = nullptr, int gm = 1,
                            const float *cs = nullptr, const float *cz = nullptr);
// The tile kernel for scale groups of 32 or 64 rows (group-aligned weights).
hipError_t launch_gemm_tile_gs(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                               const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E, int dt,
                               int group_size, hipStream_t stream, const float *cs = nullptr,
                               const float *cz = nullptr);
// Grouped gate/up projection (N = 2 * I weight columns) with the
// SiLU-and-multiply epilogue, a [M][I]; hipErrorNotSupported for tile shapes
// without a gate/up pair per wave.
hipError_t launch_gemm_tile_silu(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                                 const void *scale, const void *zero, void *a, int64_t M, int64_t K, int64_t N,
                                 int64_t E, int dt, hipStream_t stream);

// MSD: decomposition, int8 products + merge, split-K reduction.
struct MsdPlan {
    int mt;            // 16-row x tiles per workgroup (1, 2 or 4)
    int mchunks;       // workgroups along M
    int64_t mpad;      // padded row count = mchunks * 16 * mt
    int nb;            // 16-column blocks per wave
    int waves;         // waves per workgroup
    int ksplit;        // K slices (workgroups along K)
    int64_t gps;       // groups per K slice
    size_t off_coef, off_lsum, off_amax, off_layers, off_part, total;
};
MsdPlan msd_plan(int64_t M, int64_t K, int64_t N);
size_t msd_workspace_bytes(int64_t M, int64_t K, int64_t N);
int msd_config_count();
void set_msd_config(int idx);
hipError_t launch_msd(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                      int64_t N, void *workspace, hipStream_t stream);
// The same call with the workspace in the library's per-device static scratch
// (kMsdScratchBytes); hipErrorInvalidValue when the plan that runs needs more
// (msd_noalloc_bytes: the workspace of that plan alone, not the maximum over
// configurations that msd_workspace_bytes gives).
constexpr size_t kMsdScratchBytes = size_t(32) << 20;
size_t msd_noalloc_bytes(int64_t M, int64_t K, int64_t N);
hipError_t launch_msd_noalloc(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                              int64_t N, hipStream_t stream);
// Basic MSD pipeline (integer products through memory, separate merge).
size_t msd_basic_workspace_bytes(int64_t M, int64_t K, int64_t N);
hipError_t launch_msd_basic(const void *x, const void *wp, const void *scale, void *y, int64_t M, int64_t K,
                            int64_t N, void *workspace, hipStream_t stream);
hipError_t launch_msd_intermediates(const void *x, const void *wp, int64_t M, int64_t K, int64_t N,
                                    float *amax, int8_t *layers, int32_t *yint, void *workspace,
                                    hipStream_t stream);

// MoE fused-experts chain: routing prep, gather, SiLU-and-multiply, weighted
// sum, and the whole chain around two grouped GEMMs.
constexpr int kMoeMaxExperts = 1024;
struct MoePlan {
    size_t off_offsets, off_row_of, off_tok, off_h, off_a, off_o, total;
};
MoePlan moe_plan(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I);
hipError_t launch_moe_align(const int32_t *ids, int64_t T, int64_t topk, int64_t E, int32_t *offsets,
                            int32_t *sorted, int32_t *row_of, hipStream_t stream, int32_t *tok_of_row = nullptr);
hipError_t launch_moe_gather(const void *x, const int32_t *sorted, const int32_t *offsets, int64_t T,
                             int64_t topk, int64_t E, int64_t H, void *xs, hipStream_t stream);
hipError_t launch_silu_and_mul(const void *h, const int32_t *row_count, int64_t R, int64_t I, void *a, int dt,
                               hipStream_t stream);
hipError_t launch_moe_sum(const void *o, const int32_t *row_of, const float *topk_w, int64_t T, int64_t topk,
                          int64_t N, void *out, int dt, hipStream_t stream);
hipError_t launch_fused_moe(const void *x, const int32_t *ids, const float *topk_w, const void *w13, const void *s13,
                            const void *z13, const void *w2, const void *s2, const void *z2, void *out, int64_t T,
                            int64_t topk, int64_t E, int64_t H, int64_t I, int dt, void *workspace,
                            hipStream_t stream);

// W4A8-MXFP4: weight prepack (1088-byte tiles), MXFP8 activation
// quantization, and the small-M GEMM (x != nullptr: activations quantized in
// registers; else read prequantized from qx / sx).
size_t mx_prepacked_bytes(int64_t E, int64_t K, int64_t N);
hipError_t launch_mx_prepack(const void *w, const void *sw, void *out, int64_t E, int64_t K, int64_t N,
                             hipStream_t stream);
hipError_t launch_mx_quantize(const void *x, void *qx, void *sx, int64_t M, int64_t K, int dt, hipStream_t stream);
int mx_small_config_count();
void set_mx_small_config(int idx);
int64_t mx_small_max_k();
hipError_t launch_mx_gemm_small(const void *x, const void *qx, const void *sx, const void *wp, void *y, int64_t M,
                                int64_t K, int64_t N, int dt, hipStream_t stream);
// Large-M tile kernel from prequantized activations (sx 4-byte aligned);
// grouped (MoE) when offsets != nullptr (then M = R routed rows, E experts).
int mx_tile_config_count();
void set_mx_tile_config(int idx);
hipError_t launch_mx_gemm_tile(const void *qx, const void *sx, const void *wp, void *y, int64_t M, int64_t K,
                               int64_t N, int dt, hipStream_t stream, const int32_t *offsets = nullptr,
                               int64_t E = 1);

// W8A16: 8-bit weight prepack (2048-byte tiles) and the dense GEMM (small:
// split-K kernel for M <= 16 and K <= w8_small_max_k(); else the tile kernel).
size_t w8_prepacked_bytes(int64_t E, int64_t K, int64_t N);
hipError_t launch_w8_prepack(const void *w, void *out, int64_t E, int64_t K, int64_t N, int is_signed,
                             hipStream_t stream);
int64_t w8_small_max_k();
int w8_small_config_count();
void set_w8_small_config(int idx);
int w8_tile_config_count();
void set_w8_tile_config(int idx);
hipError_t launch_w8_gemm(const void *x, const void *wp, const void *scale, const void *zero, void *y, int64_t M,
                          int64_t K, int64_t N, int dt, int gm, bool small, hipStream_t stream,
                          const float *cs = nullptr, const float *cz = nullptr);

// Floating-point zero points: S (row sums per scale group) and the fp32
// correction C[M][N] in the workspace; *corr receives C for the epilogue.
size_t fzero_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t gs);
hipError_t launch_fzero_corr(const void *x, const void *scale, const void *zf, int64_t M, int64_t K, int64_t N,
                             int64_t gs, int bits, int dt, void *workspace, float **corr, hipStream_t stream);

}  // namespace w4
