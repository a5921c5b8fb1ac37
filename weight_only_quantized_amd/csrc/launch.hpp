// launch.hpp — internal launchers between the C-ABI layer (api.cpp) and the
// kernels.  All pointers are device pointers; shapes were validated by the
// caller.  Each launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

hipError_t launch_prepack(const void *w, void *out, int64_t E, int64_t K, int64_t N, int is_signed,
                          hipStream_t stream);
hipError_t launch_unpack(const void *in, void *w, int64_t E, int64_t K, int64_t N, int is_signed,
                         hipStream_t stream);

// Small-M split-K kernel (M <= 16, K <= small_max_k()).
int small_config_count();
void set_small_config(int idx);
int64_t small_max_k();
hipError_t launch_gemm_small(const void *x, const void *wp, const void *scale, const void *zero, void *y,
                             int64_t M, int64_t K, int64_t N, int dt, hipStream_t stream);

// LDS-staged tile kernel; grouped when offsets != nullptr (then M = R rows).
int tile_config_count();
void set_tile_config(int idx);
hipError_t launch_gemm_tile(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                            const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E,
                            int dt, hipStream_t stream);

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
hipError_t launch_msd_intermediates(const void *x, const void *wp, int64_t M, int64_t K, int64_t N,
                                    float *amax, int8_t *layers, int32_t *yint, void *workspace,
                                    hipStream_t stream);

}  // namespace w4
