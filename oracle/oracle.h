/*
 * oracle.h — CPU oracle for the weight-only quantized matmul (W4A16, group
 * 128) and its MSD (multi-step decomposition) variant.
 *
 * TEST INFRASTRUCTURE.  This is a plain, slow, obviously-correct host
 * implementation used only to check the HIP library.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load or
 * call it.  It shares no code, header, table or helper with the HIP library:
 * both sides only consume the same seeded input bytes.
 *
 * All pointers are HOST pointers.  Layouts are the plain user layouts:
 *   x      [M][K]      16-bit patterns (fp16 or bf16), row-major
 *   w      [K][N/2]    int4, two per byte along N, low nibble = even n;
 *                       signed two's complement when zero == NULL,
 *                       unsigned 0..15 otherwise
 *   scale  [G][N]      16-bit patterns, same dtype as x, G = K/group
 *   zero   [G][N/2]    unsigned int4 packed like w (nullable)
 *   y      [M][N]      16-bit patterns, same dtype as x
 *
 * Sources (cited by page title and section):
 *  - "WeightQuantBatchMatmulExperiment operator deep-dive: MSD algorithm for
 *    A16W4 PerGroup pseudo-quant MatMul" (CANN ops-nn sample), §4.1 eqs. 1-11
 *    (MSD), §4.2 (operator spec: fp16 x / int4 weight / fp16 antiquant_scale ->
 *    fp16 y), §4.3 (two int4 per byte, scale shape (K/128, N)).
 *  - "Humming: open-source library for quantized inference" (vLLM / Ant
 *    Group article), section on the standard quantization descriptor
 *    (group INT4 weights, scale granularity, zero points).
 */
#ifndef W4A16_ORACLE_H
#define W4A16_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

int oracle_num_threads(void);
void oracle_set_num_threads(int n);

/* Exact decoding of 16-bit float patterns and round-to-nearest-even encoding. */
double   oracle_f16_to_double(uint16_t h);
double   oracle_bf16_to_double(uint16_t b);
uint16_t oracle_double_to_f16(double v);
uint16_t oracle_double_to_bf16(double v);
void     oracle_round_array(const double *v, uint16_t *out, int64_t n, int dtype);

/* Dense: y64[m][n] = sum_k x[m][k] * (q[k][n] - z[g(k)][n]) * s[g(k)][n]  (fp64),
 * y = RNE(y64) in the dtype of x.  y64 or y may be NULL. */
void oracle_w4a16(const uint16_t *x, const uint8_t *w, const uint16_t *scale,
                  const uint8_t *zero, int64_t M, int64_t K, int64_t N,
                  int64_t group, int dtype, double *y64, uint16_t *y);

/* Same definition evaluated only at P points (rows[p], cols[p]); fp64 out. */
void oracle_w4a16_points(const uint16_t *x, const uint8_t *w, const uint16_t *scale,
                         const uint8_t *zero, int64_t M, int64_t K, int64_t N,
                         int64_t group, int dtype, const int64_t *rows,
                         const int64_t *cols, int64_t P, double *out);

/* Grouped (MoE): rows offsets[e]..offsets[e+1] of x use expert e's weights
 * w + e*K*N/2, scale + e*G*N, zero + e*G*N/2. */
void oracle_grouped(const uint16_t *x, const int32_t *offsets, const uint8_t *w,
                    const uint16_t *scale, const uint8_t *zero, int64_t E, int64_t R,
                    int64_t K, int64_t N, int64_t group, int dtype,
                    double *y64, uint16_t *y);

/* MSD, step by step.  x, scale are fp16; weights signed int4. */
void oracle_msd_amax(const uint16_t *x, int64_t M, int64_t K, int64_t group, float *amax /*[M][G]*/);
void oracle_msd_layers(const uint16_t *x, const float *amax, int64_t M, int64_t K,
                       int64_t group, int8_t *layers /*[3][M][K]*/);
void oracle_msd_decompose_one(float a, float amax, int8_t out[3], float t_out[3]);
void oracle_msd_yint(const int8_t *layers, const uint8_t *w, int64_t M, int64_t K,
                     int64_t N, int64_t group, int32_t *yint /*[G][3][M][N]*/);
void oracle_msd(const uint16_t *x, const uint8_t *w, const uint16_t *scale, int64_t M,
                int64_t K, int64_t N, int64_t group, double *y64, uint16_t *y,
                float *amax_out /*nullable [M][G]*/, int8_t *layers_out /*nullable [3][M][K]*/);

/* Reference of the prepacked weight layout (the library's own format, stated
 * in words in the design notes) and its inverse.  w/out sizes E*K*N/2. */
void oracle_prepack(const uint8_t *w, uint8_t *packed, int64_t E, int64_t K, int64_t N, int is_signed);
void oracle_unpack(const uint8_t *packed, uint8_t *w, int64_t E, int64_t K, int64_t N, int is_signed);
/* The same with a layout selector: 0 as above, 1 the group-aligned layout for
 * scale groups of 32 or 64 rows (word t of slot L holds rows
 * 128*g + 32*t + 8*(L/16) + i). */
void oracle_prepack_layout(const uint8_t *w, uint8_t *packed, int64_t E, int64_t K, int64_t N, int is_signed,
                           int layout);
void oracle_unpack_layout(const uint8_t *packed, uint8_t *w, int64_t E, int64_t K, int64_t N, int is_signed,
                          int layout);

/* ---- MoE fused-experts chain (pwwt.cn notes, §5: fused_experts_impl runs
 * moe_gemm -> fuse_silu_mul -> moe_gemm; FlagGems-vLLM operator list, MoE and
 * activation tables: moe_align_block_size, silu_and_mul, moe_sum).  Routing
 * entry i = t*topk + k of token t picks expert topk_ids[i] with weight
 * topk_w[i] (fp32); ids outside [0, E) are not routed. ---- */

/* Routing prep: routed entries ordered by (expert, i) and numbered
 * r = 0..R-1; offsets[e] = routed entries with expert < e (offsets[E] = R),
 * sorted[r] = i of row r (R entries written), row_of[i] = r, or -1 when
 * entry i is not routed.  Returns R. */
int64_t oracle_moe_align(const int32_t *topk_ids, int64_t T, int64_t topk, int64_t E,
                         int32_t *offsets, int32_t *sorted, int32_t *row_of);

/* a[r][i] = RNE( silu(h[r][i]) * h[r][I + i] ), silu(g) = g / (1 + exp(-g)),
 * in fp64; h is [R][2I] (gate half first), a is [R][I], dtype of both. */
void oracle_silu_and_mul(const uint16_t *h, int64_t R, int64_t I, int dtype, uint16_t *a);

/* out[t][n] = RNE( sum over routed k, ascending, of topk_w[t*topk+k] *
 * o[row_of[t*topk+k]][n] ) in fp64; a token with no routed entry gets 0. */
void oracle_moe_sum(const uint16_t *o, const int32_t *row_of, const float *topk_w,
                    int64_t T, int64_t topk, int64_t N, int dtype, uint16_t *out);

/* The whole chain for tokens tok[0..P-1]:
 *   h   = RNE(x[t] . dequant(W13_e))            [2I]   (W13_e: [H][2I])
 *   a   = silu_and_mul(h)                       [I]
 *   o   = RNE(a . dequant(W2_e))                [H]    (W2_e: [I][H])
 *   out[p] = RNE( sum_k topk_w[t,k] * o_k )     [H]
 * with e = topk_ids[t*topk+k] over the routed k, the weights in the plain
 * layouts (w13 [E][H][I], s13 [E][H/128][2I], z13 [E][H/128][I] or NULL;
 * w2 [E][I][H/2], s2 [E][I/128][H], z2 [E][I/128][H/2] or NULL). */
void oracle_fused_moe(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                      const uint8_t *w13, const uint16_t *s13, const uint8_t *z13,
                      const uint8_t *w2, const uint16_t *s2, const uint8_t *z2,
                      int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I,
                      int64_t group, int dtype, const int64_t *tok, int64_t P, uint16_t *out);

/* ---- W4A16 with floating-point zero points (Humming article: the
 * descriptor's zero points, here as values of the activation dtype):
 * dequant(W)[k][n] = (u[k][n] - zf[k/group][n]) * s[k/group][n], u the
 * unsigned 4-bit code, zf [K/group][N] 16-bit patterns of dtype.  fp64 sums
 * (every term exact), y = RNE(y64). ---- */
void oracle_w4a16_fzero(const uint16_t *x, const uint8_t *w, const uint16_t *scale, const uint16_t *zf,
                        int64_t M, int64_t K, int64_t N, int64_t group, int dtype, double *y64, uint16_t *y);

/* ---- W8A16 (Humming article: the WNA16 setting with N = 8, i.e. 8-bit integer
 * weights with 16-bit activations, group scales and optional zero points).
 * w[K][N] one byte per weight: two's complement int8 when zero == NULL, else
 * uint8 with uint8 zero points zero[K/group][N]; scale[K/group][N] in dtype.
 * y64 = x . ((q - z) * s) in fp64 (every product exact), y = RNE(y64). ---- */
void oracle_w8a16(const uint16_t *x, const uint8_t *w, const uint16_t *scale, const uint8_t *zero,
                  int64_t M, int64_t K, int64_t N, int64_t group, int dtype, double *y64, uint16_t *y);
/* W8A16 with floating-point zero points: (u - zf[k/group][n]) * s, u uint8,
 * zf 16-bit patterns of dtype. */
void oracle_w8a16_fzero(const uint16_t *x, const uint8_t *w, const uint16_t *scale, const uint16_t *zf,
                        int64_t M, int64_t K, int64_t N, int64_t group, int dtype, double *y64, uint16_t *y);

/* ---- W4A8-MXFP4 (Humming article: W4A8-MXFP4 path; formats per the OCP
 * Microscaling (MX) specification v1.0: blocks of 32 elements along K sharing
 * one power-of-two E8M0 scale).  Weights: E2M1 codes w[K][N/2] (two per byte
 * along N, low nibble = even n) with scales sw[K/32][N]; activations:
 * quantized to MXFP8 (E4M3 codes qx[M][K], scales sx[M][K/32]). ---- */
double oracle_e4m3_to_double(uint8_t v);     /* OCP E4M3 (bias 7, no infinities, 0x7F/0xFF NaN) */
double oracle_e2m1_to_double(uint8_t v);     /* OCP E2M1: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} */
double oracle_e8m0_to_double(uint8_t v);     /* 2^(v - 127), 0xFF NaN */

/* MXFP8 quantization of one row-block set: for each row m and 32-block b,
 * shared exponent e = floor(log2(max |x|)) - 8 (8 = largest E4M3 exponent),
 * clamped to [-127, 127] (an all-zero block gets e = -127); scale byte e + 127;
 * element = E4M3 round-to-nearest-even of x / 2^e, saturated to +-448. */
void oracle_mxfp8_quantize(const uint16_t *x, int64_t M, int64_t K, int dtype, uint8_t *qx, uint8_t *sx);

/* y64[m][n] = sum_k E4M3(qx[m][k]) 2^(sx[m][k/32]-127) * E2M1(w[k][n]) 2^(sw[k/32][n]-127)
 * in fp64 (every product exact), y = RNE(y64) in dtype (y64 or y may be NULL). */
void oracle_w4a8_mxfp4(const uint8_t *qx, const uint8_t *sx, const uint8_t *w, const uint8_t *sw,
                       int64_t M, int64_t K, int64_t N, int dtype, double *y64, uint16_t *y);

#ifdef __cplusplus
}
#endif
#endif
