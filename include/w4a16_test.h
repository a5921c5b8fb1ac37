/*
 * w4a16_test.h — test hooks of libw4a16.  Not part of the product API: they
 * expose intermediate results of the same kernels for bit-exact checks on
 * small shapes, and let tests force a kernel variant.
 */
#ifndef W4A16_TEST_H
#define W4A16_TEST_H

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Inverse of w4a16_prepack: w_packed -> plain w[E][K][N/2] (device pointers). */
w4a16_status w4a16_test_unpack(const void *w_packed, void *w, int64_t E, int64_t K, int64_t N,
                               int is_signed, void *stream);

/*
 * MSD intermediates from the production kernels (small shapes only):
 *   amax    [M][K/128]      fp32  (eq.1)
 *   layers  [3][M][K]       int8  (eqs.2-8), plain k order
 *   yint    [K/128][3][M][N] int32 (eq.9), one product per group
 * workspace as for w4a16_msd_gemm.  All pointers are device pointers.
 */
w4a16_status w4a16_test_msd_intermediates(const void *x, const void *w_packed, int64_t M,
                                          int64_t K, int64_t N, int64_t group_size,
                                          float *amax, int8_t *layers, int32_t *yint,
                                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * The MSD page's basic pipeline (§6.1 stage order with the per-group integer
 * products written to memory, as its Y_int workspace does, then a separate
 * merge kernel), for comparison with w4a16_msd_gemm, whose merge is fused
 * into the product kernel so the products never leave registers.  Same
 * arguments and result definition as w4a16_msd_gemm; the workspace (size from
 * the query below) also holds Y_int [K/128][3][M][N] int32.  scale and y need
 * 8-byte alignment.  Benchmarks and tests only.
 */
size_t w4a16_test_msd_basic_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);
w4a16_status w4a16_test_msd_basic(const void *x, const void *w_packed, const void *antiquant_scale, void *y,
                                  int64_t M, int64_t K, int64_t N, int64_t group_size, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Force the dense GEMM kernel family for subsequent calls in this process:
 * 0 = automatic (default), 1 = small-M split-K kernel, 2 = tile kernel.
 * Not thread-safe; tests and benchmarks only.  Returns the previous value.
 */
int w4a16_test_force_variant(int variant);

/*
 * Select the (column blocks, groups per wave) configuration of the small-M
 * kernel for subsequent calls with M <= 16: idx in [0, count), or -1 for the
 * default (its two-tile form for 16 < M <= 64 always takes the shape that
 * fits 8 waves).  Tuning only; not thread-safe.  Returns the number of
 * configurations.
 */
int w4a16_test_small_config(int idx);

/*
 * Select the workgroup tile configuration (rows x columns, waves) of the
 * tile kernel, dense and grouped, for subsequent calls: idx in [0, count),
 * or -1 for the default.  Tuning only; not thread-safe.  Returns the number
 * of configurations.
 */
int w4a16_test_tile_config(int idx);

/*
 * Half items of the grouped tile kernel (32-row tiles of four waves): with
 * enable = 0, subsequent grouped calls run every item over the whole K range
 * in one wave per column tile, so every output is accumulated in the same
 * order under every tile configuration; enable = 1 restores the default
 * (the item plan may split an item's K range between two wave pairs).
 * Tuning and tests only; not thread-safe.  Returns the previous setting.
 */
int w4a16_test_tile_halves(int enable);

/*
 * Select the configuration (row tiles per workgroup, column blocks per wave,
 * waves) of the MSD product kernel for subsequent calls: idx in [0, count), or
 * -1 for the default.  w4a16_msd_workspace_bytes() covers every configuration.
 * Tuning only; not thread-safe.  Returns the number of configurations.
 */
int w4a16_test_msd_config(int idx);

/* Select the W4A8-MXFP4 small-M kernel variant (-1 = automatic); returns the
 * number of variants. */
int w4a16_test_mx_small_config(int idx);

/* Select the W8A16 small-M and tile kernel variants (-1 = automatic);
 * returns 100 * (small variants) + (tile variants).  w4a16_test_force_variant(2)
 * also forces W8A16 calls onto the tile kernel. */
int w4a16_test_w8_config(int small_idx, int tile_idx);

/* Select the W4A8-MXFP4 tile kernel variant (-1 = automatic); returns the
 * number of variants.  w4a16_test_force_variant(2) also forces the W4A8-MXFP4
 * calls onto the tile kernel (and then w4a8_mxfp4_workspace_bytes asks for
 * a workspace at every M). */
int w4a16_test_mx_tile_config(int idx);

/* Name of the kernel variant the dispatcher picks for a dense call. */
const char *w4a16_test_variant_name(int64_t M, int64_t K, int64_t N, int dt, int has_zero);

#ifdef __cplusplus
}
#endif
#endif
