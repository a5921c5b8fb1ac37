/*
 * w4a16.h — libw4a16: weight-only quantized matrix multiply on AMD Instinct
 * MI355X (gfx950, CDNA4).  Plain C ABI: device pointers, sizes, a stream.
 *
 * Computes Y = X . dequant(W) with
 *   X     fp16 or bf16 activations,
 *   W     int4 weights, one scale (same dtype as X) and optionally one uint4
 *         zero point per group of `group_size` consecutive K rows and per
 *         column (group_size 32, 64 or a multiple of 128; group_size == K
 *         gives one scale per column),
 *   dequant(W)[k][n] = (q[k][n] - z[k/gs][n]) * s[k/gs][n], gs = group_size,
 *   fp32 accumulation, Y rounded to the dtype of X.
 * Sources: "Humming: open-source library for quantized inference" (vLLM /
 * Ant Group article), section on the standard quantization descriptor (group
 * INT4 weights with BF16 activations, scale granularity, zero points);
 * "WeightQuantBatchMatmulExperiment operator deep-dive: MSD algorithm for
 * A16W4 PerGroup pseudo-quant MatMul" (CANN ops-nn sample), §4.2 operator
 * spec and §4.3 data layout (two int4 per byte, scale shape (K/128, N)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *    on the current HIP device.  `stream` is a hipStream_t (NULL = the
 *    default stream).  Work is enqueued asynchronously; no call synchronizes
 *    or allocates device memory.
 *  - Plain weight layout: w[E][K][N/2] bytes; element (k, n) is nibble
 *    (n & 1) of byte k*N/2 + n/2 (low nibble = even n).
 *  - Signedness: when `zero` is NULL the weights are signed two's-complement
 *    int4 in [-8, 7] and MUST have been prepacked with is_signed = 1; when
 *    `zero` is given the weights are unsigned in [0, 15] (prepacked with
 *    is_signed = 0) and zero[G][N/2] holds uint4 zero points packed like w.
 *  - Shape rules: K > 0, K % 128 == 0, N > 0, N % 64 == 0, M (or R) >= 0,
 *    E >= 1.  group_size: 32, 64, or a multiple of 128 dividing K for
 *    w4a16_gemm and w4a16_grouped_gemm (else W4A16_ERR_UNSUPPORTED, or
 *    W4A16_ERR_SHAPE when it does not divide K); 32 and 64 need weights
 *    prepacked by w4a16_prepack_g with that group size; exactly 128 for the
 *    MSD path (whose page fixes the group at 128 rows) and the MoE chain.  M == 0 (or an expert without rows) is a
 *    no-op that returns W4A16_OK.
 *  - Alignment: x, w_packed, workspace 16 bytes; scale, y 2 bytes.
 *  - Errors: every argument is checked on the host before anything is
 *    enqueued; on error nothing is launched and y is untouched.  A launch
 *    failure reported by the runtime maps to W4A16_ERR_DEVICE, as does a
 *    current device that is not gfx950.  Faults inside a kernel surface, as
 *    usual in HIP, at the caller's next synchronization.
 *  - Thread safety: calls are stateless apart from a per-device property
 *    cache filled once; concurrent calls on different streams are safe.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,         /* a required pointer is NULL               */
    W4A16_ERR_SHAPE = 2,        /* a size violates the shape rules          */
    W4A16_ERR_UNSUPPORTED = 3,  /* group_size or dtype not supported        */
    W4A16_ERR_ALIGN = 4,        /* a pointer is not aligned as required     */
    W4A16_ERR_WORKSPACE = 5,    /* MSD workspace missing or too small       */
    W4A16_ERR_DEVICE = 6,       /* not a gfx950 device, or a launch failed  */
    W4A16_ERR_SCRATCH = 7       /* needs more than the static scratch holds */
} w4a16_status;

typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1 } w4a16_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *w4a16_status_str(int status);

/* Bytes of the prepacked buffer for E experts of K x N weights: E*K*N/2. */
size_t w4a16_prepacked_bytes(int64_t E, int64_t K, int64_t N);

/*
 * Offline weight repack (run once per model load).  Reorders the nibbles of
 * w[E][K][N/2] into the library's tile layout so the GEMM kernels read 32
 * nibbles of one column with one 128-bit load and dequantize them in
 * registers straight into the matrix-core operand, with no LDS round trip.
 * Layout: 1024-byte tiles ordered (expert, 16-column block, 128-row group);
 * slot L (16 bytes) of a tile holds column 16*nb + L%16, rows
 * 128*g + 32*(L/16) + r (r = 0..31); word t of the slot holds r = 8t + i with
 * row r's code at bit 4*(i/2) + 16*(i%2); the code is u (is_signed == 0) or
 * q + 8 (is_signed == 1).  Motivation: "Marlin layout" (pwwt.cn notes,
 * §6.2: weights reordered for memory access, kernels matched to the layout);
 * QUICK abstract (offline interleave that skips the shared-memory write-back
 * after dequantization); Humming article (weights reordered for the target
 * kernel).  w and w_packed: device, E*K*N/2 bytes each, must not overlap.
 */
w4a16_status w4a16_prepack(const void *w, void *w_packed, int64_t E, int64_t K, int64_t N,
                           int is_signed, void *stream);

/*
 * Weight repack for a given scale group size (Humming article: the
 * quantization descriptor keeps the scale granularity as its own parameter).
 * group_size a multiple of 128 gives exactly w4a16_prepack's layout.
 * group_size 32 or 64 gives the group-aligned layout that w4a16_gemm,
 * w4a16_grouped_gemm and w4a16_gemm_desc require for those group sizes: the
 * same tiles and slots with the roles of the slot's 32-row chunk and word
 * exchanged (word t of slot L holds rows 128*g + 32*t + 8*(L/16) + i, code
 * of row i at bit 4*(i/2) + 16*(i%2)), so each 16x16x32 and each pair of
 * 32x32x16 matrix-core steps takes the rows of one 32-row block, which lies
 * in one scale group.  Same sizes, pointers and errors as w4a16_prepack
 * (W4A16_ERR_UNSUPPORTED for another group_size, W4A16_ERR_SHAPE when it
 * does not divide K).
 */
w4a16_status w4a16_prepack_g(const void *w, void *w_packed, int64_t E, int64_t K, int64_t N,
                             int is_signed, int64_t group_size, void *stream);

/*
 * Dense W4A16 GEMM: y[M][N] = x[M][K] . dequant(W).
 *   x        [M][K] fp16/bf16 (dtype dt)
 *   w_packed prepacked weights (E = 1)
 *   scale    [K/group_size][N], dtype dt
 *   zero     [K/group_size][N/2] uint4 or NULL (see Signedness)
 *   y        [M][N], dtype dt
 * M <= 16 (K <= 8192), and 16 < M <= 64 with K <= 4096 (two 16-row tiles
 * per workgroup, 32-row groups on the grid), run a split-K matrix-core kernel
 * whose waves reduce through LDS; larger M runs an LDS-staged tile kernel
 * whose tile shape follows M.  With group_size 32 or 64 (weights from
 * w4a16_prepack_g) the split-K kernel covers M <= 16 with K <= 4096 and the
 * tile kernel the rest, each running one accumulation chain per scale group.
 */
w4a16_status w4a16_gemm(const void *x, const void *w_packed, const void *scale,
                        const void *zero, void *y, int64_t M, int64_t K, int64_t N,
                        int64_t group_size, int dt, void *stream);

/*
 * MSD A16W4 PerGroup GEMM (WeightQuantBatchMatmulExperiment operator
 * deep-dive, §4.1 eqs. 1-11): per row and 128-group, A_max = max|x|; the
 * group is split into three int4 residual layers with the fp32 factors
 * 7.49, 14.98, 14.98 (round half to even); the layers are multiplied with the
 * int4 weights by int8 matrix-core instructions with int32 accumulation, then
 * merged as ((Y1/7.49 + Y2/(7.49*14.98) + Y3/(7.49*14.98^2)) * A_max) * scale
 * and accumulated over groups in fp32.  A single row (M = 1) runs as one
 * launch that decomposes x itself and leaves the workspace untouched (it is
 * still required, as for any M); larger M runs the decomposition, the
 * product kernel over K slices and their sum.
 *   x                [M][K] fp16
 *   w_packed         prepacked signed weights (is_signed = 1)
 *   antiquant_scale  [K/128][N] fp16
 *   y                [M][N] fp16
 *   workspace        device scratch of at least w4a16_msd_workspace_bytes()
 *                    bytes, 16-byte aligned, owned by the caller; its contents
 *                    on entry are ignored and on return are unspecified.
 * Two-stage use as in the page's aclnn API (§5.4): query the size, allocate,
 * then call.  Calls sharing one workspace must be ordered on one stream.
 */
size_t w4a16_msd_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);

w4a16_status w4a16_msd_gemm(const void *x, const void *w_packed, const void *antiquant_scale,
                            void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a16_msd_gemm without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and kernels as
 * w4a16_msd_gemm; the workspace is a static device array inside the library,
 * W4A16_MSD_SCRATCH_BYTES per GPU, held by every GPU the library runs on until
 * the process ends.  A problem whose workspace (that of the kernel
 * configuration the call runs, at most w4a16_msd_workspace_bytes()) exceeds
 * it returns W4A16_ERR_SCRATCH before anything is enqueued; the shapes of the
 * MSD page fit (M = 64, K = N = 8192 needs about 19 MB; a single row needs
 * none).  Calls no allocating routine.  Every call on one GPU shares that GPU's array: calls
 * that may overlap in time on one GPU (different streams without ordering,
 * other threads) race and must be serialized by the caller.
 */
#define W4A16_MSD_SCRATCH_BYTES ((size_t)32 << 20)

w4a16_status w4a16_msd_gemm_noalloc(const void *x, const void *w_packed, const void *antiquant_scale,
                                    void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                                    void *stream);

/*
 * Grouped (MoE) W4A16 GEMM: for each expert e, rows
 * expert_offsets[e] .. expert_offsets[e+1]-1 of x are multiplied by expert
 * e's weights.  Rows must already be gathered and sorted by expert.
 *   x               [R][K], dtype dt
 *   expert_offsets  DEVICE int32[E+1], offsets[0] = 0, non-decreasing,
 *                   offsets[E] = R (read on the device only: no host sync)
 *   w_packed        prepacked weights of all E experts (E*K*N/2 bytes)
 *   scale           [E][K/group_size][N], dtype dt
 *   zero            [E][K/group_size][N/2] or NULL
 *   y               [R][N], dtype dt; rows of experts without rows: none
 * Experts with no rows cost nothing beyond a skipped tile slot (Humming
 * article: dense and MoE workloads share the kernel components).
 */
w4a16_status w4a16_grouped_gemm(const void *x, const int32_t *expert_offsets, const void *w_packed,
                                const void *scale, const void *zero, void *y, int64_t E,
                                int64_t R, int64_t K, int64_t N, int64_t group_size, int dt,
                                void *stream);

/*
 * ---- MoE fused-experts chain ---------------------------------------------
 * The chain named by the pages: an expert GEMM, a fused SiLU-and-multiply
 * and a second expert GEMM (pwwt.cn notes, §5, lmslim's fused_experts_impl),
 * with the routing prep and the weighted sum of the experts' outputs
 * (FlagGems-vLLM operator list, MoE table: moe_align_block_size, moe_sum;
 * activation table: silu_and_mul).  Routing entry i = t*topk + k of token t
 * selects expert topk_ids[i] (int32) with weight topk_w[i] (fp32); an id
 * outside [0, E) is not routed and contributes nothing.  Requires
 * 1 <= E <= 1024, topk >= 1, T*topk < 2^31.  Every device pointer below is
 * 4-byte aligned (int/float arrays) or 16-byte aligned (16-bit tensors).
 */

/*
 * Routing prep: routed entries ordered by (expert, entry index), numbered
 * r = 0..R-1 (a stable counting sort, so the result is unique).
 *   topk_ids        [T][topk] int32
 *   expert_offsets  out, int32[E+1]: rows of expert e are
 *                   offsets[e] .. offsets[e+1]-1, offsets[E] = R
 *   sorted_ids      out, int32[T*topk]: entry index of row r (r < R)
 *   row_of          out, int32[T*topk]: row of entry i, or -1 if not routed
 */
w4a16_status w4a16_moe_align(const int32_t *topk_ids, int64_t T, int64_t topk, int64_t E,
                             int32_t *expert_offsets, int32_t *sorted_ids, int32_t *row_of, void *stream);

/*
 * x_sorted[r] = x[sorted_ids[r] / topk] for the routed rows r < offsets[E]
 * (read on the device).  x [T][H], x_sorted [T*topk][H], dtype dt;
 * H % 8 == 0.
 */
w4a16_status w4a16_moe_gather(const void *x, const int32_t *sorted_ids, const int32_t *expert_offsets,
                              int64_t T, int64_t topk, int64_t E, int64_t H, void *x_sorted, int dt,
                              void *stream);

/*
 * a[r][i] = silu(h[r][i]) * h[r][I + i], silu(g) = g / (1 + exp(-g)), in
 * fp32, rounded once to dt (FlagGems-vLLM operator list, activation table:
 * SiLU activation combined with an elementwise multiply; the gate is the
 * first half).  h [R][2I], a [R][I]; I % 8 == 0.  row_count, if not NULL, is
 * a DEVICE int32 holding the number of rows to process (at most R), e.g.
 * expert_offsets + E.
 */
w4a16_status w4a16_silu_and_mul(const void *h, const int32_t *row_count, int64_t R, int64_t I, void *a,
                                int dt, void *stream);

/*
 * out[t][n] = sum over routed k (ascending) of topk_w[t][k] * o[row_of[t*topk+k]][n],
 * in fp32, rounded once to dt (FlagGems-vLLM operator list, MoE table:
 * sum of the experts' outputs).  o [rows][N], out [T][N]; N % 8 == 0.
 */
w4a16_status w4a16_moe_sum(const void *o, const int32_t *row_of, const float *topk_w, int64_t T, int64_t topk,
                           int64_t N, void *out, int dt, void *stream);

/* Workspace of w4a16_fused_moe: offsets, the row of every routing entry, the
 * token of every routed row and the intermediates h [T*topk][2I],
 * a [T*topk][I], o [T*topk][H].  0 for invalid sizes. */
size_t w4a16_fused_moe_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I);

/*
 * The whole chain for T tokens of width H through experts of width I:
 *   h = x[token of row] . dequant(W13_e)  (grouped W4A16 over the routed
 *                                    rows, which read their token's x row
 *                                    directly; W13_e [H][2I], gate columns
 *                                    first), rounded to dt
 *   a = silu_and_mul(h)              rounded to dt
 *   o = a . dequant(W2_e)            (grouped W4A16; W2_e [I][H]), rounded to dt
 *   out[t] = moe_sum(o)              [T][H], dt
 * The first two lines run as one kernel: h is rounded to dt in registers and
 * a is formed in the projection's epilogue, bit-identical to the separate
 * steps (the h part of the workspace is then unused).
 * w13_packed / w2_packed are the prepacked weights of all E experts (K = H,
 * N = 2I and K = I, N = H); s13 [E][H/128][2I], s2 [E][I/128][H] in dt;
 * z13 [E][H/128][I], z2 [E][I/128][H/2] uint4 zero points or both NULL
 * (signedness as in w4a16_gemm).  Needs H % 128 == 0, I % 128 == 0.
 * The workspace (at least w4a16_fused_moe_workspace_bytes) is used
 * asynchronously; calls sharing one must be ordered on one stream.
 */
w4a16_status w4a16_fused_moe(const void *x, const int32_t *topk_ids, const float *topk_w,
                             const void *w13_packed, const void *s13, const void *z13,
                             const void *w2_packed, const void *s2, const void *z2, void *out,
                             int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I, int64_t group_size,
                             int dt, void *workspace, size_t workspace_bytes, void *stream);

/*
 * W8A16 ("Humming: open-source library for quantized inference", the WNA16
 * setting of its quantization descriptor with 8-bit weights): as the W4A16
 * GEMM with 8-bit codes,
 *   dequant(W)[k][n] = (q[k][n] - z[k/gs][n]) * s[k/gs][n],
 *   w[E][K][N] one byte per weight: two's complement int8 q (zero == NULL,
 *   prepacked with is_signed = 1) or uint8 q with uint8 zero points
 *   zero[K/gs][N] (one byte each; is_signed = 0); scale[K/gs][N] in dt.
 * Shape, group and alignment rules as for w4a16_gemm (group_size a multiple
 * of 128 dividing K).  M <= 48 with K <= 8192 runs a split-K kernel (one
 * 16-row tile per grid row), larger M an LDS-staged tile kernel.
 */

/* Bytes of the prepacked 8-bit buffer: E*K*N. */
size_t w8a16_prepacked_bytes(int64_t E, int64_t K, int64_t N);

/*
 * Offline repack of w[E][K][N] into 2048-byte tiles ordered (expert, 16-column
 * block nb, 128-row group g): bytes 32L..32L+31 of a tile hold column
 * 16*nb + L%16, rows 128*g + 32*(L/16) + r as byte r, the code being q + 128
 * (is_signed = 1) or q.  Device pointers, E*K*N bytes each, no overlap.
 */
w4a16_status w8a16_prepack(const void *w, void *w_packed, int64_t E, int64_t K, int64_t N, int is_signed,
                           void *stream);

/* y[M][N] = x[M][K] . dequant(W) for 8-bit weights (E = 1); see above. */
w4a16_status w8a16_gemm(const void *x, const void *w_packed, const void *scale, const void *zero, void *y,
                        int64_t M, int64_t K, int64_t N, int64_t group_size, int dt, void *stream);

/*
 * Weight descriptor ("Humming: open-source library for quantized inference":
 * its standard quantization descriptor keeps apart the weight format, the
 * scale granularity, the scales' data type, the zero points and optional
 * secondary scales).  One entry point for the dense integer-weight GEMMs:
 *   dequant(W)[k][n] = (q[k][n] - z[k/gs][n]) * s[k/gs][n] * t[n]
 * with t the optional secondary scale (one fp32 value per output column,
 * applied to the fp32 sum before the one rounding; t = 1 when absent) and z
 * integer codes or floating-point values (zero_format).
 */
typedef struct {
    int32_t weight_bits;         /* 4 (prepacked by w4a16_prepack) or 8 (w8a16_prepack)             */
    int32_t zero_format;         /* 0: integer zero points (or none); 1: floating-point zero points */
    int64_t group_size;          /* rows per scale group: a multiple of 128 dividing K              */
    const void *scale;           /* [K/group_size][N], dtype of x                                   */
    const void *zero;            /* zero_format 0: NULL (signed weights) or uint4 [K/gs][N/2] packed
                                    like the weights (4-bit) / uint8 [K/gs][N] (8-bit);
                                    zero_format 1: [K/gs][N] values of the dtype of x, with the
                                    weights unsigned codes (prepacked with is_signed = 0)           */
    const float *channel_scale;  /* NULL or [N] fp32 secondary scale t                              */
} w4a16_weight_desc;

/* Scratch for w4a16_gemm_desc: 0 unless zero_format == 1 (then fp32 row sums
 * per scale group and an fp32 [M][N] correction). */
size_t w4a16_gemm_desc_workspace_bytes(const w4a16_weight_desc *desc, int64_t M, int64_t K, int64_t N);

/* y[M][N] = x[M][K] . dequant(W) as described by *desc (device pointers
 * inside it; channel_scale 4-byte aligned); otherwise as w4a16_gemm /
 * w8a16_gemm.  Floating-point zero points: the signed path multiplies the
 * codes as u - 8 (4-bit) or u - 128 (8-bit), a correction kernel forms
 * sum_g S[m][g] * (z[g][n] - 8 or 128) * s[g][n] into the workspace (S: row
 * sums of x per scale group), and the GEMM epilogue subtracts it before the
 * secondary scale and the rounding; requires K/group_size <= 8192 and
 * M <= 1048560.  workspace: >= w4a16_gemm_desc_workspace_bytes() bytes,
 * 16-byte aligned (may be NULL when that is 0); calls sharing it must be
 * ordered on one stream.  W4A16_ERR_UNSUPPORTED for another weight_bits or
 * zero_format. */
w4a16_status w4a16_gemm_desc(const void *x, const void *w_packed, const w4a16_weight_desc *desc, void *y,
                             int64_t M, int64_t K, int64_t N, int dt, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * W4A8-MXFP4 ("Humming: open-source library for quantized inference", the
 * W4A8-MXFP4 path: MXFP4 weights with 8-bit activations, aimed at small-M
 * speed; the W4A8 configuration in its list of supported weight/activation
 * settings).  Formats follow the OCP Microscaling (MX) v1.0 specification:
 *   weights      E2M1 codes w[E][K][N/2] (two per byte along N, low nibble =
 *                even n, the plain layout above) with E8M0 scales
 *                w_scale[E][K/32][N]: value = e2m1(code) * 2^(scale - 127);
 *   activations  MXFP8: E4M3 codes qx[M][K] with E8M0 scales sx[M][K/32]; a
 *                block's shared exponent is floor(log2 max|x|) - 8, clamped to
 *                [-127, 127], and each element is x / 2^e rounded to nearest
 *                even and saturated to +-448 (finite inputs only);
 *   y[m][n] = sum_k qx * 2^(sx - 127) * w * 2^(w_scale - 127), fp32
 *   accumulation, rounded to dt (fp16 or bf16).
 * gfx950's block-scaled matrix-core instruction takes both formats and both
 * scales directly; the article's in-kernel weight conversion (needed on GPUs
 * without MXFP4 matrix cores) is not needed here.
 * Shape rules: K % 128 == 0, N % 64 == 0, M >= 0, E >= 1, and one expert's
 * packed weights below 2 GiB ((K/128) * (N/16) * 1088 < 2^31).
 * Alignment: x, qx, w, w_packed, workspace 16 bytes; sx 4 bytes; y 2 bytes.
 * Kernels: M <= 48 with K <= 8192 runs a split-K kernel (one 16-row tile per
 * grid row); everything else a tile kernel that stages the quantized
 * activations in LDS.
 */

/* Bytes of the prepacked MXFP4 buffer: E * (K/128) * (N/16) * 1088. */
size_t w4a8_mxfp4_prepacked_bytes(int64_t E, int64_t K, int64_t N);

/*
 * Offline repack of MXFP4 weights and their scales into 1088-byte tiles
 * ordered (expert, 16-column block, 128-row group): bytes 16L..16L+15 of a
 * tile hold column 16*nb + L%16, rows 128*g + 32*(L/16) + r (r = 0..31) as
 * nibble r (low nibble first); byte 1024 + L holds the scale of that column
 * for rows 128*g + 32*(L/16) .. +31.  This is the block-scaled instruction's
 * own operand order, so one 128-bit and one 8-bit load per lane feed it.
 * w: E*K*N/2 bytes, w_scale: E*(K/32)*N bytes, w_packed:
 * w4a8_mxfp4_prepacked_bytes() bytes; device pointers, no overlap.
 */
w4a16_status w4a8_mxfp4_prepack(const void *w, const void *w_scale, void *w_packed, int64_t E, int64_t K,
                                int64_t N, void *stream);

/* MXFP8 quantization of activations x[M][K] (dtype dt) into qx[M][K] (E4M3)
 * and sx[M][K/32] (E8M0), as defined above.  Bit-exact by construction. */
w4a16_status w4a8_mxfp8_quantize(const void *x, void *qx, void *sx, int64_t M, int64_t K, int dt, void *stream);

/* y[M][N] (dtype dt) from prequantized MXFP8 activations and prepacked
 * MXFP4 weights (E = 1). */
w4a16_status w4a8_mxfp4_gemm_prequant(const void *qx, const void *sx, const void *w_packed, void *y, int64_t M,
                                      int64_t K, int64_t N, int dt, void *stream);

/* Scratch for w4a8_mxfp4_gemm: room for qx and sx (M*K bytes rounded up to
 * 256, then M*K/32), whichever kernel the call picks, so one query always
 * suffices.  The split-K kernel (M <= 48, K <= 8192: activations quantized in
 * its registers) uses none of it, and for those calls the workspace may be
 * NULL.  Returns 0 for M <= 0 or K <= 0. */
size_t w4a8_mxfp4_workspace_bytes(int64_t M, int64_t K);

/*
 * y[M][N] = MXFP8(x) . MXFP4(W): quantizes x (dtype dt) and multiplies.  For
 * M <= 48 (K <= 8192) one kernel does both (each wave quantizes its K slice
 * in registers); otherwise x is quantized into the workspace first.
 * workspace: device, >= w4a8_mxfp4_workspace_bytes(M, K) bytes, or NULL for
 * a call that runs the split-K kernel (W4A16_ERR_WORKSPACE if the tile kernel
 * runs without one); contents on return unspecified; calls sharing one
 * workspace must be ordered on one stream.
 */
w4a16_status w4a8_mxfp4_gemm(const void *x, const void *w_packed, void *y, int64_t M, int64_t K, int64_t N,
                             int dt, void *workspace, size_t workspace_bytes, void *stream);

/* Scratch for w4a8_mxfp4_grouped_gemm: room for the MXFP8 codes and scales of
 * all R rows. */
size_t w4a8_mxfp4_grouped_workspace_bytes(int64_t R, int64_t K);

/*
 * Grouped (MoE) W4A8-MXFP4: rows expert_offsets[e] .. expert_offsets[e+1]-1
 * of x are multiplied by expert e's MXFP4 weights (the Humming article runs
 * dense and MoE layers on the same kernel components).  x [R][K] (dtype dt),
 * rows already gathered and sorted by expert; expert_offsets DEVICE
 * int32[E+1] as for w4a16_grouped_gemm (read on the device only); w_packed
 * the E experts' prepacked weights; y [R][N].  The R rows are quantized to
 * MXFP8 into the workspace (>= w4a8_mxfp4_grouped_workspace_bytes(R, K),
 * 16-byte aligned; contents on return unspecified; calls sharing it must be
 * ordered on one stream), then one grouped tile kernel runs.
 */
w4a16_status w4a8_mxfp4_grouped_gemm(const void *x, const int32_t *expert_offsets, const void *w_packed, void *y,
                                     int64_t E, int64_t R, int64_t K, int64_t N, int dt, void *workspace,
                                     size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
