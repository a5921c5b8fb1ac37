// api.cpp — C ABI of libw4a16: argument validation, device check, dispatch.
// Every check runs on the host before any launch (nothing is enqueued on an
// error).  No exception crosses the ABI; the library never allocates device
// memory and never synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/w4a16.h"
#include "../../include/w4a16_test.h"
#include "launch.hpp"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    std::once_flag once;
    bool gfx950 = false;
    int cus = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::atomic<int> g_force_variant{0};

// 1 if the current device is gfx950, 0 if not, -1 on a runtime error.
int current_device_ok() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    DeviceInfo &d = g_dev[dev];
    std::call_once(d.once, [&] {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.cus = prop.multiProcessorCount;
        }
    });
    return d.gfx950 ? 1 : 0;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

w4a16_status map_err(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_DEVICE; }

w4a16_status check_kn(int64_t K, int64_t N, int64_t group_size) {
    if (group_size != 128) return W4A16_ERR_UNSUPPORTED;
    if (K <= 0 || N <= 0 || K % 128 != 0 || N % 64 != 0) return W4A16_ERR_SHAPE;
    // the kernels index tiles and rows with 32-bit grid coordinates
    if (K > (int64_t(1) << 30) || N > (int64_t(1) << 30)) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// Scale groups for the dense and grouped GEMMs: any multiple of 128 that
// divides K (group_size == K is one scale per column).  On success *gm is the
// number of 128-row groups per scale group.
w4a16_status check_kn_groups(int64_t K, int64_t N, int64_t group_size, int *gm) {
    if (group_size < 128 || group_size % 128 != 0) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_kn(K, N, 128);
    if (st != W4A16_OK) return st;
    if (K % group_size != 0) return W4A16_ERR_SHAPE;
    *gm = (int)(group_size / 128);
    return W4A16_OK;
}

// Scale groups of 32 or 64 rows (the group-aligned weight layout): *gr is the
// group size; W4A16_ERR_UNSUPPORTED for other sizes below 128.
w4a16_status check_kn_small_groups(int64_t K, int64_t N, int64_t group_size, int *gr) {
    if (group_size != 32 && group_size != 64) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_kn(K, N, 128);
    if (st != W4A16_OK) return st;
    *gr = (int)group_size;
    return W4A16_OK;
}

// W4A8-MXFP4 shapes: K a multiple of 128 up to the small kernel's K limit,
// N a multiple of 64.
// The packed weights of one expert are addressed with 32-bit byte offsets.
w4a16_status check_mx_kn(int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K % 128 != 0 || N % 64 != 0) return W4A16_ERR_SHAPE;
    if (K > (int64_t(1) << 30) || N > (int64_t(1) << 30)) return W4A16_ERR_SHAPE;
    if ((K / 128) * (N / 16) * 1088 > (int64_t(1) << 31) - 1) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// Row limit of the MXFP4 GEMM (32-bit row tiles on the first grid axis).
constexpr int64_t kMxMaxM = (int64_t(1) << 31) - 1;

// MXFP4 dispatch: M <= 48 (and K within the split-K kernel's reach) runs the
// split-K kernel, one 16-row tile per grid row (measured at K = 4096,
// N = 14336: M = 24/32/48 in 15.5/16.8/23.1 us against 26.4/27.0/26.4 us on
// the tile kernel, M = 64 in 29.3 against 26.8 us), everything else the tile
// kernel; the test hook can force the tile kernel.
bool mx_use_small(int64_t M, int64_t K) {
    const int forced = g_force_variant.load(std::memory_order_relaxed);
    if (forced == 2) return false;
    return M <= 48 && K <= w4::mx_small_max_k();
}

// Offset of sx behind qx in the W4A8-MXFP4 workspace (256-byte aligned).
size_t mx_ws_sx_offset(int64_t M, int64_t K) { return ((size_t)M * (size_t)K + 255) & ~(size_t)255; }

// W8A16: the split-K kernel (one 16-row tile per grid row) up to M = 48
// (measured at K = 4096, N = 14336: M = 24/32/48 in 22.2/24.1/33.0 us against
// 37.4/38.6/40.4 us on the tile kernel; M = 64 42.2 against 40.4 us).
constexpr int64_t kW8SmallMaxM = 48;

// Dense dispatch table: decode-sized M goes to the split-K kernel (one 16-row
// tile up to M = 16; with K <= 4096 two, and a second pair of tiles on the
// grid up to M = 64), the rest to the LDS-staged tile kernel.
int pick_variant(int64_t M, int64_t K) {
    const bool small_ok = (M <= 16 && K <= w4::small_max_k()) || (M <= 64 && K <= w4::small2_max_k());
    const int forced = g_force_variant.load(std::memory_order_relaxed);
    if (forced == 1 && small_ok) return 1;
    if (forced == 2) return 2;
    return small_ok ? 1 : 2;
}

}  // namespace

extern "C" {

const char *w4a16_status_str(int status) {
    switch (status) {
        case W4A16_OK: return "W4A16_OK";
        case W4A16_ERR_NULL: return "W4A16_ERR_NULL: a required pointer is NULL";
        case W4A16_ERR_SHAPE: return "W4A16_ERR_SHAPE: sizes violate K>0, K%128==0, N>0, N%64==0, M>=0, E>=1";
        case W4A16_ERR_UNSUPPORTED: return "W4A16_ERR_UNSUPPORTED: group_size must be 32, 64 or a multiple of 128 (MSD and the MoE chain: 128; W8A16 and floating-point zero points: a multiple of 128), dtype F16 or BF16 (MSD: F16)";
        case W4A16_ERR_ALIGN: return "W4A16_ERR_ALIGN: x, w_packed, workspace need 16-byte, scale and y 2-byte alignment";
        case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE: MSD workspace is NULL or smaller than w4a16_msd_workspace_bytes()";
        case W4A16_ERR_DEVICE: return "W4A16_ERR_DEVICE: current device is not gfx950 or a launch failed";
        case W4A16_ERR_SCRATCH:
            return "W4A16_ERR_SCRATCH: the problem needs more workspace than the library's static scratch "
                   "(W4A16_MSD_SCRATCH_BYTES); use w4a16_msd_gemm with a caller workspace";
        default: return "W4A16_ERR_UNKNOWN";
    }
}

size_t w4a16_prepacked_bytes(int64_t E, int64_t K, int64_t N) {
    if (E < 1 || K <= 0 || N <= 0) return 0;
    return (size_t)E * (size_t)K * (size_t)N / 2;
}

w4a16_status w4a16_prepack(const void *w, void *w_packed, int64_t E, int64_t K, int64_t N, int is_signed,
                           void *stream) {
    if (!w || !w_packed) return W4A16_ERR_NULL;
    if (E < 1) return W4A16_ERR_SHAPE;
    w4a16_status st = check_kn(K, N, 128);
    if (st != W4A16_OK) return st;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_prepack(w, w_packed, E, K, N, is_signed ? 1 : 0, (hipStream_t)stream));
}

w4a16_status w4a16_prepack_g(const void *w, void *w_packed, int64_t E, int64_t K, int64_t N, int is_signed,
                             int64_t group_size, void *stream) {
    if (!w || !w_packed) return W4A16_ERR_NULL;
    if (E < 1) return W4A16_ERR_SHAPE;
    int layout = 0, gx = 1;
    w4a16_status st = group_size < 128 ? check_kn_small_groups(K, N, group_size, &gx)
                                       : check_kn_groups(K, N, group_size, &gx);
    if (st != W4A16_OK) return st;
    if (group_size < 128) layout = 1;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_prepack(w, w_packed, E, K, N, is_signed ? 1 : 0, (hipStream_t)stream, layout));
}

// Dense call with 32- or 64-row scale groups (group-aligned weights).
static w4a16_status gemm_small_groups(const void *x, const void *w_packed, const void *scale, const void *zero,
                                      void *y, int64_t M, int64_t K, int64_t N, int gr, int dt, hipStream_t s,
                                      const float *cs) {
    const int forced = g_force_variant.load(std::memory_order_relaxed);
    if (forced != 2 && M <= 16 && K <= w4::small_gs_max_k())
        return map_err(w4::launch_gemm_small_gs(x, w_packed, scale, zero, y, M, K, N, dt, gr, s, cs));
    return map_err(w4::launch_gemm_tile_gs(x, nullptr, w_packed, scale, zero, y, M, K, N, 1, dt, gr, s, cs));
}

w4a16_status w4a16_gemm(const void *x, const void *w_packed, const void *scale, const void *zero, void *y,
                        int64_t M, int64_t K, int64_t N, int64_t group_size, int dt, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    int gm = 1, gr = 0;
    w4a16_status st = group_size < 128 ? check_kn_small_groups(K, N, group_size, &gr)
                                       : check_kn_groups(K, N, group_size, &gm);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > (int64_t(1) << 31) - 1) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !w_packed || !scale || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(scale, 2) || !aligned(y, 2))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    hipStream_t s = (hipStream_t)stream;
    if (gr) return gemm_small_groups(x, w_packed, scale, zero, y, M, K, N, gr, dt, s, nullptr);
    if (pick_variant(M, K) == 1)
        return map_err(w4::launch_gemm_small(x, w_packed, scale, zero, y, M, K, N, dt, s, gm));
    return map_err(w4::launch_gemm_tile(x, nullptr, w_packed, scale, zero, y, M, K, N, 1, dt, s, nullptr, gm));
}

size_t w4a16_msd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size) {
    if (check_kn(K, N, group_size) != W4A16_OK || M < 0) return 0;
    if (M == 0) return 0;
    return w4::msd_workspace_bytes(M, K, N);
}

w4a16_status w4a16_msd_gemm(const void *x, const void *w_packed, const void *antiquant_scale, void *y,
                            int64_t M, int64_t K, int64_t N, int64_t group_size, void *workspace,
                            size_t workspace_bytes, void *stream) {
    w4a16_status st = check_kn(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > (int64_t(1) << 24)) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !w_packed || !antiquant_scale || !y) return W4A16_ERR_NULL;
    if (!workspace || workspace_bytes < w4::msd_workspace_bytes(M, K, N)) return W4A16_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(antiquant_scale, 2) || !aligned(y, 16) ||
        !aligned(workspace, 16))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_msd(x, w_packed, antiquant_scale, y, M, K, N, workspace, (hipStream_t)stream));
}

w4a16_status w4a16_msd_gemm_noalloc(const void *x, const void *w_packed, const void *antiquant_scale, void *y,
                                    int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream) {
    w4a16_status st = check_kn(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > (int64_t(1) << 24)) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !w_packed || !antiquant_scale || !y) return W4A16_ERR_NULL;
    if (w4::msd_noalloc_bytes(M, K, N) > w4::kMsdScratchBytes) return W4A16_ERR_SCRATCH;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(antiquant_scale, 2) || !aligned(y, 16))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_msd_noalloc(x, w_packed, antiquant_scale, y, M, K, N, (hipStream_t)stream));
}

w4a16_status w4a16_grouped_gemm(const void *x, const int32_t *expert_offsets, const void *w_packed,
                                const void *scale, const void *zero, void *y, int64_t E, int64_t R, int64_t K,
                                int64_t N, int64_t group_size, int dt, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    int gm = 1, gr = 0;
    w4a16_status st = group_size < 128 ? check_kn_small_groups(K, N, group_size, &gr)
                                       : check_kn_groups(K, N, group_size, &gm);
    if (st != W4A16_OK) return st;
    if (E < 1 || E > (int64_t(1) << 20) || R < 0 || R > (int64_t(1) << 31) - 1) return W4A16_ERR_SHAPE;
    if (R == 0) return W4A16_OK;
    if (!x || !expert_offsets || !w_packed || !scale || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(scale, 2) || !aligned(y, 2) ||
        !aligned(expert_offsets, 4))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    if (gr)
        return map_err(w4::launch_gemm_tile_gs(x, expert_offsets, w_packed, scale, zero, y, R, K, N, E, dt, gr,
                                               (hipStream_t)stream));
    return map_err(w4::launch_gemm_tile(x, expert_offsets, w_packed, scale, zero, y, R, K, N, E, dt,
                                        (hipStream_t)stream, nullptr, gm));
}

// ---- MoE fused-experts chain -------------------------------------------------

}  // extern "C"

namespace {

w4a16_status check_route(int64_t T, int64_t topk, int64_t E) {
    if (T < 0 || topk < 1 || E < 1) return W4A16_ERR_SHAPE;
    if (E > w4::kMoeMaxExperts) return W4A16_ERR_UNSUPPORTED;
    if (topk > (int64_t(1) << 20) || T > (int64_t(1) << 31) / topk - 1) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

bool dt_ok(int dt) { return dt == W4A16_F16 || dt == W4A16_BF16; }

}  // namespace

extern "C" {

w4a16_status w4a16_moe_align(const int32_t *topk_ids, int64_t T, int64_t topk, int64_t E,
                             int32_t *expert_offsets, int32_t *sorted_ids, int32_t *row_of, void *stream) {
    w4a16_status st = check_route(T, topk, E);
    if (st != W4A16_OK) return st;
    if (!expert_offsets || (T > 0 && (!topk_ids || !sorted_ids || !row_of))) return W4A16_ERR_NULL;
    if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_ids, 4) || !aligned(row_of, 4))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_moe_align(topk_ids, T, topk, E, expert_offsets, sorted_ids, row_of,
                                        (hipStream_t)stream));
}

w4a16_status w4a16_moe_gather(const void *x, const int32_t *sorted_ids, const int32_t *expert_offsets,
                              int64_t T, int64_t topk, int64_t E, int64_t H, void *x_sorted, int dt,
                              void *stream) {
    if (!dt_ok(dt)) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_route(T, topk, E);
    if (st != W4A16_OK) return st;
    if (H <= 0 || H % 8 != 0 || H > (int64_t(1) << 30)) return W4A16_ERR_SHAPE;
    if (T == 0) return W4A16_OK;
    if (!x || !sorted_ids || !expert_offsets || !x_sorted) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(x_sorted, 16) || !aligned(sorted_ids, 4) || !aligned(expert_offsets, 4))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_moe_gather(x, sorted_ids, expert_offsets, T, topk, E, H, x_sorted,
                                         (hipStream_t)stream));
}

w4a16_status w4a16_silu_and_mul(const void *h, const int32_t *row_count, int64_t R, int64_t I, void *a,
                                int dt, void *stream) {
    if (!dt_ok(dt)) return W4A16_ERR_UNSUPPORTED;
    if (R < 0 || I <= 0 || I % 8 != 0 || I > (int64_t(1) << 30) || R > (int64_t(1) << 31)) return W4A16_ERR_SHAPE;
    if (R == 0) return W4A16_OK;
    if (!h || !a) return W4A16_ERR_NULL;
    if (!aligned(h, 16) || !aligned(a, 16) || !aligned(row_count, 4)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_silu_and_mul(h, row_count, R, I, a, dt, (hipStream_t)stream));
}

w4a16_status w4a16_moe_sum(const void *o, const int32_t *row_of, const float *topk_w, int64_t T, int64_t topk,
                           int64_t N, void *out, int dt, void *stream) {
    if (!dt_ok(dt)) return W4A16_ERR_UNSUPPORTED;
    if (T < 0 || topk < 1 || topk > (int64_t(1) << 20) || T > (int64_t(1) << 31) / topk - 1) return W4A16_ERR_SHAPE;
    if (N <= 0 || N % 8 != 0 || N > (int64_t(1) << 30)) return W4A16_ERR_SHAPE;
    if (T == 0) return W4A16_OK;
    if (!o || !row_of || !topk_w || !out) return W4A16_ERR_NULL;
    if (!aligned(o, 16) || !aligned(out, 16) || !aligned(row_of, 4) || !aligned(topk_w, 4)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_moe_sum(o, row_of, topk_w, T, topk, N, out, dt, (hipStream_t)stream));
}

size_t w4a16_fused_moe_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I) {
    if (check_route(T, topk, E) != W4A16_OK) return 0;
    if (check_kn(H, 2 * I, 128) != W4A16_OK || check_kn(I, H, 128) != W4A16_OK) return 0;
    return w4::moe_plan(T, topk, E, H, I).total;
}

w4a16_status w4a16_fused_moe(const void *x, const int32_t *topk_ids, const float *topk_w,
                             const void *w13_packed, const void *s13, const void *z13,
                             const void *w2_packed, const void *s2, const void *z2, void *out,
                             int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I, int64_t group_size,
                             int dt, void *workspace, size_t workspace_bytes, void *stream) {
    if (!dt_ok(dt)) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_route(T, topk, E);
    if (st != W4A16_OK) return st;
    // gate/up: K = H, N = 2I; down: K = I, N = H
    if ((st = check_kn(H, 2 * I, group_size)) != W4A16_OK) return st;
    if ((st = check_kn(I, H, group_size)) != W4A16_OK) return st;
    if ((z13 == nullptr) != (z2 == nullptr)) return W4A16_ERR_NULL;
    if (T == 0) return W4A16_OK;
    if (!x || !topk_ids || !topk_w || !w13_packed || !s13 || !w2_packed || !s2 || !out) return W4A16_ERR_NULL;
    if (!workspace || workspace_bytes < w4::moe_plan(T, topk, E, H, I).total) return W4A16_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w13_packed, 16) || !aligned(w2_packed, 16) ||
        !aligned(workspace, 16) || !aligned(s13, 2) || !aligned(s2, 2) || !aligned(topk_ids, 4) ||
        !aligned(topk_w, 4))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_fused_moe(x, topk_ids, topk_w, w13_packed, s13, z13, w2_packed, s2, z2, out, T, topk,
                                        E, H, I, dt, workspace, (hipStream_t)stream));
}

// ---- test hooks -------------------------------------------------------------

w4a16_status w4a16_test_unpack(const void *w_packed, void *w, int64_t E, int64_t K, int64_t N, int is_signed,
                               void *stream) {
    if (!w || !w_packed) return W4A16_ERR_NULL;
    if (E < 1) return W4A16_ERR_SHAPE;
    w4a16_status st = check_kn(K, N, 128);
    if (st != W4A16_OK) return st;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_unpack(w_packed, w, E, K, N, is_signed ? 1 : 0, (hipStream_t)stream));
}

w4a16_status w4a16_test_msd_intermediates(const void *x, const void *w_packed, int64_t M, int64_t K, int64_t N,
                                          int64_t group_size, float *amax, int8_t *layers, int32_t *yint,
                                          void *workspace, size_t workspace_bytes, void *stream) {
    w4a16_status st = check_kn(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (M <= 0 || M > 4096) return W4A16_ERR_SHAPE;
    if (!x || !w_packed || !amax || !layers || !yint) return W4A16_ERR_NULL;
    if (!workspace || workspace_bytes < w4::msd_workspace_bytes(M, K, N)) return W4A16_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(workspace, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_msd_intermediates(x, w_packed, M, K, N, amax, layers, yint, workspace,
                                                (hipStream_t)stream));
}

size_t w4a16_test_msd_basic_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size) {
    if (check_kn(K, N, group_size) != W4A16_OK || M <= 0 || M > (int64_t(1) << 24)) return 0;
    return w4::msd_basic_workspace_bytes(M, K, N);
}

w4a16_status w4a16_test_msd_basic(const void *x, const void *w_packed, const void *antiquant_scale, void *y,
                                  int64_t M, int64_t K, int64_t N, int64_t group_size, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    w4a16_status st = check_kn(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > (int64_t(1) << 24)) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !w_packed || !antiquant_scale || !y) return W4A16_ERR_NULL;
    if (!workspace || workspace_bytes < w4::msd_basic_workspace_bytes(M, K, N)) return W4A16_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(antiquant_scale, 8) || !aligned(y, 8) ||
        !aligned(workspace, 16))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_msd_basic(x, w_packed, antiquant_scale, y, M, K, N, workspace, (hipStream_t)stream));
}

int w4a16_test_force_variant(int variant) { return g_force_variant.exchange(variant); }

const char *w4a16_test_variant_name(int64_t M, int64_t K, int64_t N, int dt, int has_zero) {
    (void)N; (void)dt; (void)has_zero;
    return pick_variant(M, K) == 1 ? "gemm_small_kernel" : "gemm_tile_kernel";
}

int w4a16_test_small_config(int idx) {
    w4::set_small_config(idx);
    return w4::small_config_count();
}

int w4a16_test_tile_config(int idx) {
    w4::set_tile_config(idx);
    return w4::tile_config_count();
}

int w4a16_test_tile_halves(int enable) { return w4::set_tile_halves(enable); }

int w4a16_test_msd_config(int idx) {
    w4::set_msd_config(idx);
    return w4::msd_config_count();
}

int w4a16_test_mx_small_config(int idx) {
    w4::set_mx_small_config(idx);
    return w4::mx_small_config_count();
}

int w4a16_test_w8_config(int small_idx, int tile_idx) {
    w4::set_w8_small_config(small_idx);
    w4::set_w8_tile_config(tile_idx);
    return w4::w8_small_config_count() * 100 + w4::w8_tile_config_count();
}

// ---- W8A16 ------------------------------------------------------------------

size_t w8a16_prepacked_bytes(int64_t E, int64_t K, int64_t N) {
    if (E < 1 || K <= 0 || N <= 0) return 0;
    return w4::w8_prepacked_bytes(E, K, N);
}

w4a16_status w8a16_prepack(const void *w, void *w_packed, int64_t E, int64_t K, int64_t N, int is_signed,
                           void *stream) {
    if (E < 1) return W4A16_ERR_SHAPE;
    w4a16_status st = check_kn(K, N, 128);
    if (st != W4A16_OK) return st;
    if (!w || !w_packed) return W4A16_ERR_NULL;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_w8_prepack(w, w_packed, E, K, N, is_signed ? 1 : 0, (hipStream_t)stream));
}

w4a16_status w8a16_gemm(const void *x, const void *w_packed, const void *scale, const void *zero, void *y,
                        int64_t M, int64_t K, int64_t N, int64_t group_size, int dt, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    int gm = 1;
    w4a16_status st = check_kn_groups(K, N, group_size, &gm);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > (int64_t(1) << 31) - 1) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !w_packed || !scale || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(scale, 2) || !aligned(y, 2))
        return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    const int forced = g_force_variant.load(std::memory_order_relaxed);
    const bool small = forced != 2 && M <= kW8SmallMaxM && K <= w4::w8_small_max_k();
    return map_err(w4::launch_w8_gemm(x, w_packed, scale, zero, y, M, K, N, dt, gm, small, (hipStream_t)stream));
}

size_t w4a8_mxfp4_grouped_workspace_bytes(int64_t R, int64_t K) {
    if (R <= 0 || K <= 0) return 0;
    return mx_ws_sx_offset(R, K) + (size_t)R * (size_t)(K / 32);
}

w4a16_status w4a8_mxfp4_grouped_gemm(const void *x, const int32_t *expert_offsets, const void *w_packed, void *y,
                                     int64_t E, int64_t R, int64_t K, int64_t N, int dt, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_mx_kn(K, N);
    if (st != W4A16_OK) return st;
    if (E < 1 || E > (int64_t(1) << 20) || R < 0 || R > kMxMaxM) return W4A16_ERR_SHAPE;
    if (R == 0) return W4A16_OK;
    if (!x || !expert_offsets || !w_packed || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 2) || !aligned(expert_offsets, 4))
        return W4A16_ERR_ALIGN;
    const size_t need = w4a8_mxfp4_grouped_workspace_bytes(R, K);
    if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    const hipStream_t s = (hipStream_t)stream;
    uint8_t *qx = (uint8_t *)workspace;
    uint8_t *sx = qx + mx_ws_sx_offset(R, K);
    hipError_t e = w4::launch_mx_quantize(x, qx, sx, R, K, dt, s);
    if (e != hipSuccess) return map_err(e);
    return map_err(w4::launch_mx_gemm_tile(qx, sx, w_packed, y, R, K, N, dt, s, expert_offsets, E));
}

size_t w4a16_gemm_desc_workspace_bytes(const w4a16_weight_desc *desc, int64_t M, int64_t K, int64_t N) {
    if (!desc || desc->zero_format != 1 || M <= 0 || K <= 0 || N <= 0 || desc->group_size < 128 ||
        K % desc->group_size != 0)
        return 0;
    return w4::fzero_workspace_bytes(M, K, N, desc->group_size);
}

w4a16_status w4a16_gemm_desc(const void *x, const void *w_packed, const w4a16_weight_desc *desc, void *y,
                             int64_t M, int64_t K, int64_t N, int dt, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (!desc) return W4A16_ERR_NULL;
    if ((desc->weight_bits != 4 && desc->weight_bits != 8) || (desc->zero_format != 0 && desc->zero_format != 1))
        return W4A16_ERR_UNSUPPORTED;
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    int gm = 1, gr = 0;
    // 32/64-row scale groups: 4-bit weights with integer zero points (or none)
    if (desc->group_size < 128 && (desc->weight_bits != 4 || desc->zero_format != 0)) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = desc->group_size < 128 ? check_kn_small_groups(K, N, desc->group_size, &gr)
                                             : check_kn_groups(K, N, desc->group_size, &gm);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > (int64_t(1) << 31) - 1) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    const bool fz = desc->zero_format == 1;
    if (!x || !w_packed || !desc->scale || !y || (fz && !desc->zero)) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(desc->scale, 2) || !aligned(y, 2) ||
        !aligned(desc->channel_scale, 4) || (fz && !aligned(desc->zero, 2)))
        return W4A16_ERR_ALIGN;
    if (fz) {
        if (K / desc->group_size > 8192 || M > 65535 * 16) return W4A16_ERR_SHAPE;
        if (!workspace || workspace_bytes < w4a16_gemm_desc_workspace_bytes(desc, M, K, N))
            return W4A16_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return W4A16_ERR_ALIGN;
    }
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    const hipStream_t s = (hipStream_t)stream;
    const float *cs = desc->channel_scale;
    // floating-point zero points: the signed path (zero NULL) plus the correction
    const void *zero = fz ? nullptr : desc->zero;
    float *cz = nullptr;
    if (fz) {
        hipError_t e = w4::launch_fzero_corr(x, desc->scale, desc->zero, M, K, N, desc->group_size,
                                             desc->weight_bits, dt, workspace, &cz, s);
        if (e != hipSuccess) return map_err(e);
    }
    if (desc->weight_bits == 8) {
        const int forced = g_force_variant.load(std::memory_order_relaxed);
        const bool small = forced != 2 && M <= kW8SmallMaxM && K <= w4::w8_small_max_k();
        return map_err(w4::launch_w8_gemm(x, w_packed, desc->scale, zero, y, M, K, N, dt, gm, small, s, cs, cz));
    }
    if (gr) return gemm_small_groups(x, w_packed, desc->scale, zero, y, M, K, N, gr, dt, s, cs);
    if (pick_variant(M, K) == 1)
        return map_err(w4::launch_gemm_small(x, w_packed, desc->scale, zero, y, M, K, N, dt, s, gm, cs, cz));
    return map_err(w4::launch_gemm_tile(x, nullptr, w_packed, desc->scale, zero, y, M, K, N, 1, dt, s, nullptr,
                                        gm, cs, cz));
}

int w4a16_test_mx_tile_config(int idx) {
    w4::set_mx_tile_config(idx);
    return w4::mx_tile_config_count();
}

// ---- W4A8-MXFP4 -------------------------------------------------------------

size_t w4a8_mxfp4_prepacked_bytes(int64_t E, int64_t K, int64_t N) {
    if (E < 1 || K <= 0 || N <= 0) return 0;
    return w4::mx_prepacked_bytes(E, K, N);
}

w4a16_status w4a8_mxfp4_prepack(const void *w, const void *w_scale, void *w_packed, int64_t E, int64_t K,
                                int64_t N, void *stream) {
    if (E < 1) return W4A16_ERR_SHAPE;
    w4a16_status st = check_mx_kn(K, N);
    if (st != W4A16_OK) return st;
    if (!w || !w_scale || !w_packed) return W4A16_ERR_NULL;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_mx_prepack(w, w_scale, w_packed, E, K, N, (hipStream_t)stream));
}

w4a16_status w4a8_mxfp8_quantize(const void *x, void *qx, void *sx, int64_t M, int64_t K, int dt, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    if (M < 0 || K <= 0 || K % 128 != 0 || M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 30))
        return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !qx || !sx) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(qx, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    return map_err(w4::launch_mx_quantize(x, qx, sx, M, K, dt, (hipStream_t)stream));
}

w4a16_status w4a8_mxfp4_gemm_prequant(const void *qx, const void *sx, const void *w_packed, void *y, int64_t M,
                                      int64_t K, int64_t N, int dt, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_mx_kn(K, N);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > kMxMaxM) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!qx || !sx || !w_packed || !y) return W4A16_ERR_NULL;
    if (!aligned(qx, 16) || !aligned(sx, 4) || !aligned(w_packed, 16) || !aligned(y, 2)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    const hipStream_t s = (hipStream_t)stream;
    if (mx_use_small(M, K)) return map_err(w4::launch_mx_gemm_small(nullptr, qx, sx, w_packed, y, M, K, N, dt, s));
    return map_err(w4::launch_mx_gemm_tile(qx, sx, w_packed, y, M, K, N, dt, s));
}

// Room for qx and sx: the query does not depend on which kernel a call would
// pick (nor on the test hook that forces one), so a size taken once always
// suffices; the split-K path uses none of it.
size_t w4a8_mxfp4_workspace_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return mx_ws_sx_offset(M, K) + (size_t)M * (size_t)(K / 32);
}

w4a16_status w4a8_mxfp4_gemm(const void *x, const void *w_packed, void *y, int64_t M, int64_t K, int64_t N,
                             int dt, void *workspace, size_t workspace_bytes, void *stream) {
    if (dt != W4A16_F16 && dt != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    w4a16_status st = check_mx_kn(K, N);
    if (st != W4A16_OK) return st;
    if (M < 0 || M > kMxMaxM) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !w_packed || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 2)) return W4A16_ERR_ALIGN;
    const size_t need = mx_use_small(M, K) ? 0 : w4a8_mxfp4_workspace_bytes(M, K);
    if (need > 0 && (!workspace || workspace_bytes < need)) return W4A16_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return W4A16_ERR_ALIGN;
    if (current_device_ok() != 1) return W4A16_ERR_DEVICE;
    const hipStream_t s = (hipStream_t)stream;
    if (mx_use_small(M, K)) return map_err(w4::launch_mx_gemm_small(x, nullptr, nullptr, w_packed, y, M, K, N, dt, s));
    uint8_t *qx = (uint8_t *)workspace;
    uint8_t *sx = qx + mx_ws_sx_offset(M, K);
    hipError_t e = w4::launch_mx_quantize(x, qx, sx, M, K, dt, s);
    if (e != hipSuccess) return map_err(e);
    return map_err(w4::launch_mx_gemm_tile(qx, sx, w_packed, y, M, K, N, dt, s));
}

}  // extern "C"
