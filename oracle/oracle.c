/*
 * oracle.c — CPU oracle for W4A16 (group 128) and MSD A16W4 PerGroup.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Plain loops, fp64 for the dense
 * definition, IEEE binary32 exactly as written for the MSD decomposition.
 * Build with -O2 -ffp-contract=off and without -ffast-math so that every
 * float operation rounds once, in program order (x86-64 SSE arithmetic).
 *
 * The dense/grouped result has a plain definition,
 *     Y = X . dequant(W),   dequant(W)[k][n] = (q[k][n] - z[g][n]) * s[g][n],
 * g = k / 128 (Humming article: group INT4 weights with a scale and optional
 * zero point per group; the operator spec of the MSD page §4.2 / §4.3 fixes
 * a (K/128, N) scale).  The oracle writes that definition out.
 *
 * MSD is an encoding, so its oracle follows the eleven steps of the
 * WeightQuantBatchMatmulExperiment page, §4.1, in that page's order:
 *   eq.1  A_max = rowMax(|A_group|)
 *   eq.2-7 tmp1 = 7.49*A/A_max, A1 = round(tmp1), tmp2 = (tmp1-A1)*14.98,
 *          A2 = round(tmp2), tmp3 = (tmp2-A2)*14.98, A3 = round(tmp3)
 *   eq.8-9 Y_int = [A1;A2;A3] . Weight_group   (integer matmul)
 *   eq.10  Y_group = ((Y1/7.49 + Y2/(7.49*14.98) + Y3/(7.49*14.98*14.98))*A_max)*scale_group
 *   eq.11  Y = sum over groups of Y_group
 * with the factors {7.49f, 14.98f, 14.98f} stored as fp32 constants (§4.1).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <assert.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the following parallel loops (timing runs only). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* 16-bit float decoding (exact) and RNE encoding from fp64.                  */
/* ------------------------------------------------------------------------- */

double oracle_f16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), exp - 25);   /* (1.man) * 2^(exp-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_double(uint16_t b) {
    int sign = (b >> 15) & 1;
    int exp = (b >> 7) & 0xFF;
    int man = b & 0x7F;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -133);                /* subnormal: man * 2^-133 */
    else if (exp == 255)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + man), exp - 134);   /* (1.man) * 2^(exp-127) */
    return sign ? -v : v;
}

/* Round |v| to a binary float with `mbits` explicit mantissa bits, exponent
 * bias `bias`, `ebits` exponent bits, round-to-nearest-even (rint in the
 * default rounding mode is RNE; the scalings by powers of two are exact). */
static uint16_t encode_rne(double v, int mbits, int ebits, int bias) {
    uint16_t sign = signbit(v) ? (uint16_t)(1u << (mbits + ebits)) : 0;
    double a = fabs(v);
    int emax_field = (1 << ebits) - 1;
    uint16_t inf = (uint16_t)(sign | (emax_field << mbits));
    if (isnan(v)) return (uint16_t)(inf | (1u << (mbits - 1)));
    if (isinf(a)) return inf;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1): unbiased exponent e-1 */
    int unb = e - 1;
    int emin = 1 - bias;
    if (unb < emin) {
        /* subnormal range: quantum 2^(emin - mbits) */
        double n = rint(ldexp(a, mbits - emin));
        /* n == 2^mbits rounds up into the smallest normal: same bit pattern */
        return (uint16_t)(sign | (uint16_t)n);
    }
    double n = rint(ldexp(a, mbits - unb));          /* in [2^mbits, 2^(mbits+1)] */
    if (n >= ldexp(1.0, mbits + 1)) { n = ldexp(1.0, mbits); unb += 1; }
    int field = unb + bias;
    if (field >= emax_field) return inf;
    return (uint16_t)(sign | (field << mbits) | ((uint16_t)n - (1u << mbits)));
}

uint16_t oracle_double_to_f16(double v) { return encode_rne(v, 10, 5, 15); }
uint16_t oracle_double_to_bf16(double v) { return encode_rne(v, 7, 8, 127); }

void oracle_round_array(const double *v, uint16_t *out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORACLE_BF16 ? oracle_double_to_bf16(v[i]) : oracle_double_to_f16(v[i]);
}

static double to_double(uint16_t bits, int dtype) {
    return dtype == ORACLE_BF16 ? oracle_bf16_to_double(bits) : oracle_f16_to_double(bits);
}

/* ------------------------------------------------------------------------- */
/* int4 decoding of the plain layout                                          */
/* ------------------------------------------------------------------------- */

/* 4-bit code of element (row, col) of a [rows][cols/2]-byte packed matrix. */
static int nibble(const uint8_t *p, int64_t cols, int64_t row, int64_t col) {
    uint8_t byte = p[row * (cols / 2) + col / 2];
    return (col & 1) ? (byte >> 4) : (byte & 0xF);
}

/* Integer weight value: two's complement int4 when signed, else 0..15. */
static int weight_int(const uint8_t *w, int64_t N, int64_t k, int64_t n, int is_signed) {
    int c = nibble(w, N, k, n);
    return is_signed ? (c >= 8 ? c - 16 : c) : c;
}

/* dequant(W)[k][n] = (q - z) * s, exact in fp64 (|q - z| < 2^5, s has at most
 * 11 significant bits, so the product has at most 16 bits). */
static double dequant(const uint8_t *w, const uint16_t *scale, const uint8_t *zero,
                      int64_t N, int64_t group, int dtype, int64_t k, int64_t n) {
    int64_t g = k / group;
    int is_signed = zero == NULL;
    int q = weight_int(w, N, k, n, is_signed);
    int z = zero ? nibble(zero, N, g, n) : 0;
    return (double)(q - z) * to_double(scale[g * N + n], dtype);
}

/* ------------------------------------------------------------------------- */
/* Dense W4A16                                                                */
/* ------------------------------------------------------------------------- */

void oracle_w4a16(const uint16_t *x, const uint8_t *w, const uint16_t *scale,
                  const uint8_t *zero, int64_t M, int64_t K, int64_t N,
                  int64_t group, int dtype, double *y64, uint16_t *y) {
    if (M <= 0) return;
    /* Step 1: dequant(W) materialised in fp64 (exact). */
    double *wd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    assert(wd);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            wd[k * N + n] = dequant(w, scale, zero, N, group, dtype, k, n);

    double *acc = y64 ? y64 : (double *)malloc(sizeof(double) * (size_t)M * (size_t)N);
    assert(acc);
    /* Step 2: acc[m][n] = sum_k x[m][k] * wd[k][n], each sum taken in
     * ascending k (the loops over n only run independent sums side by side). */
    const int64_t NC = 512;
    int64_t nchunks = (N + NC - 1) / NC;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NC, n1 = n0 + NC < N ? n0 + NC : N;
            double *row = acc + m * N;
            for (int64_t n = n0; n < n1; ++n) row[n] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = to_double(x[m * K + k], dtype);
                const double *wr = wd + k * N;
                for (int64_t n = n0; n < n1; ++n) row[n] += xv * wr[n];
            }
        }
    }
    /* Step 3: one rounding to the output dtype. */
    if (y) oracle_round_array(acc, y, M * N, dtype);
    if (!y64) free(acc);
    free(wd);
}

void oracle_w4a16_points(const uint16_t *x, const uint8_t *w, const uint16_t *scale,
                         const uint8_t *zero, int64_t M, int64_t K, int64_t N,
                         int64_t group, int dtype, const int64_t *rows,
                         const int64_t *cols, int64_t P, double *out) {
    (void)M;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = rows[p], n = cols[p];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += to_double(x[m * K + k], dtype) * dequant(w, scale, zero, N, group, dtype, k, n);
        out[p] = s;
    }
}

void oracle_grouped(const uint16_t *x, const int32_t *offsets, const uint8_t *w,
                    const uint16_t *scale, const uint8_t *zero, int64_t E, int64_t R,
                    int64_t K, int64_t N, int64_t group, int dtype,
                    double *y64, uint16_t *y) {
    int64_t G = K / group;
    (void)R;
    for (int64_t e = 0; e < E; ++e) {
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
        if (r1 <= r0) continue;   /* expert without rows: nothing to compute */
        oracle_w4a16(x + r0 * K, w + e * K * (N / 2), scale + e * G * N,
                     zero ? zero + e * G * (N / 2) : NULL, r1 - r0, K, N, group, dtype,
                     y64 ? y64 + r0 * N : NULL, y ? y + r0 * N : NULL);
    }
}

/* ------------------------------------------------------------------------- */
/* MSD (multi-step decomposition), step by step                               */
/* ------------------------------------------------------------------------- */

static const float MSD_F1 = 7.49f;    /* first factor  (fp32 constant) */
static const float MSD_F2 = 14.98f;   /* second/third factor            */

void oracle_msd_amax(const uint16_t *x, int64_t M, int64_t K, int64_t group, float *amax) {
    int64_t G = K / group;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g) {
            float mx = 0.0f;
            for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                float a = fabsf((float)oracle_f16_to_double(x[m * K + k]));  /* exact */
                if (a > mx) mx = a;
            }
            amax[m * G + g] = mx;   /* eq.1: rowMax(|A_group|), per row and group */
        }
}

/* eqs.2-7 for one element.  Each line is one binary32 operation, rounded to
 * nearest even; round() is round-half-to-even (rintf).  An all-zero group
 * (amax == 0) has all three layers 0. */
void oracle_msd_decompose_one(float a, float amax, int8_t out[3], float t_out[3]) {
    if (amax == 0.0f) {
        out[0] = out[1] = out[2] = 0;
        if (t_out) t_out[0] = t_out[1] = t_out[2] = 0.0f;
        return;
    }
    float p = MSD_F1 * a;          /* 7.49 * A            */
    float t1 = p / amax;           /* tmp1 = 7.49*A/A_max  (eq.2) */
    float a1 = rintf(t1);          /* A1 = round(tmp1)     (eq.3) */
    float d1 = t1 - a1;
    float t2 = d1 * MSD_F2;        /* tmp2 = (tmp1-A1)*14.98 (eq.4) */
    float a2 = rintf(t2);          /* A2 = round(tmp2)     (eq.5) */
    float d2 = t2 - a2;
    float t3 = d2 * MSD_F2;        /* tmp3 = (tmp2-A2)*14.98 (eq.6) */
    float a3 = rintf(t3);          /* A3 = round(tmp3)     (eq.7) */
    out[0] = (int8_t)a1;
    out[1] = (int8_t)a2;
    out[2] = (int8_t)a3;
    if (t_out) { t_out[0] = t1; t_out[1] = t2; t_out[2] = t3; }
}

void oracle_msd_layers(const uint16_t *x, const float *amax, int64_t M, int64_t K,
                       int64_t group, int8_t *layers) {
    int64_t G = K / group;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            int8_t l[3];
            float a = (float)oracle_f16_to_double(x[m * K + k]);
            oracle_msd_decompose_one(a, amax[m * G + k / group], l, NULL);
            for (int j = 0; j < 3; ++j) layers[(j * M + m) * K + k] = l[j];  /* eq.8: [A1;A2;A3] */
        }
}

void oracle_msd_yint(const int8_t *layers, const uint8_t *w, int64_t M, int64_t K,
                     int64_t N, int64_t group, int32_t *yint) {
    int64_t G = K / group;
    /* eq.9: Y_int = A_int . Weight_group, one integer product per group. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t g = 0; g < G; ++g)
        for (int64_t m = 0; m < M; ++m)
            for (int j = 0; j < 3; ++j)
                for (int64_t n = 0; n < N; ++n) {
                    int64_t s = 0;
                    for (int64_t k = g * group; k < (g + 1) * group; ++k)
                        s += (int64_t)layers[(j * M + m) * K + k] * weight_int(w, N, k, n, 1);
                    assert(s >= INT32_MIN && s <= INT32_MAX);
                    yint[((g * 3 + j) * M + m) * N + n] = (int32_t)s;
                }
}

void oracle_msd(const uint16_t *x, const uint8_t *w, const uint16_t *scale, int64_t M,
                int64_t K, int64_t N, int64_t group, double *y64, uint16_t *y,
                float *amax_out, int8_t *layers_out) {
    if (M <= 0) return;
    int64_t G = K / group;
    float *amax = (float *)malloc(sizeof(float) * (size_t)(M * G));
    int8_t *layers = (int8_t *)malloc((size_t)(3 * M * K));
    int8_t *q = (int8_t *)malloc((size_t)(K * N));
    double *acc = y64 ? y64 : (double *)malloc(sizeof(double) * (size_t)(M * N));
    assert(amax && layers && q && acc);

    oracle_msd_amax(x, M, K, group, amax);            /* eq.1   */
    oracle_msd_layers(x, amax, M, K, group, layers);  /* eqs.2-8 */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) q[k * N + n] = (int8_t)weight_int(w, N, k, n, 1);

    const double c1 = (double)MSD_F1, c2 = (double)MSD_F2;
#pragma omp parallel
    {
        int64_t *Y = (int64_t *)malloc(sizeof(int64_t) * (size_t)(3 * N));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            double *row = acc + m * N;
            for (int64_t n = 0; n < N; ++n) row[n] = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                /* eq.9 for this (row, group): three integer dot products per column */
                memset(Y, 0, sizeof(int64_t) * (size_t)(3 * N));
                for (int j = 0; j < 3; ++j)
                    for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                        int64_t a = layers[(j * M + m) * K + k];
                        if (a == 0) continue;
                        const int8_t *qr = q + k * N;
                        int64_t *Yj = Y + j * N;
                        for (int64_t n = 0; n < N; ++n) Yj[n] += a * (int64_t)qr[n];
                    }
                /* eq.10 (merge, fp64) and eq.11 (accumulate over groups) */
                double am = (double)amax[m * G + g];
                for (int64_t n = 0; n < N; ++n) {
                    double yg = ((double)Y[n] / c1 + (double)Y[N + n] / (c1 * c2) +
                                 (double)Y[2 * N + n] / (c1 * c2 * c2)) * am;
                    row[n] += yg * oracle_f16_to_double(scale[g * N + n]);
                }
            }
        }
        free(Y);
    }
    if (y) oracle_round_array(acc, y, M * N, ORACLE_F16);
    if (amax_out) memcpy(amax_out, amax, sizeof(float) * (size_t)(M * G));
    if (layers_out) memcpy(layers_out, layers, (size_t)(3 * M * K));
    if (!y64) free(acc);
    free(q);
    free(layers);
    free(amax);
}

/* ------------------------------------------------------------------------- */
/* Prepacked layout (the library's own format)                                */
/* ------------------------------------------------------------------------- */
/*
 * The packed buffer is a sequence of 1024-byte tiles, one per (expert e,
 * column block nb of 16 columns, K-group g of 128 rows), ordered e, nb, g.
 * Inside a tile, 16-byte slot L (0..63) holds column n = 16*nb + (L % 16) for
 * the 32 rows k = 128*g + 32*(L / 16) + r, r = 0..31.  Slot word t (0..3,
 * little-endian uint32 at byte 4t of the slot) holds r = 8t + i, i = 0..7, with
 * the 4-bit code of row r at bit 4*(i / 2) + 16*(i % 2).  The code is the
 * unsigned value u (unsigned weights) or q + 8 (signed weights q in [-8, 7]).
 *
 * Group-aligned layout (layout 1, for scale groups of 32 or 64 rows): the
 * same tiles, slots, words and bit positions, with the roles of the slot's
 * chunk c = L / 16 and the word t exchanged: word t of slot L holds the rows
 * k = 128*g + 32*t + 8*c + i, i = 0..7.  (Layout 0 above is the case
 * k = 128*g + 32*c + 8*t + i.)
 */
static int64_t packed_bit_index(int64_t K, int64_t N, int64_t e, int64_t k, int64_t n, int layout) {
    int64_t G = K / 128, NB = N / 16;
    int64_t nb = n / 16, j = n % 16, g = k / 128, kk = k % 128;
    int64_t c, t, i = kk % 8;
    if (layout == 1) {
        t = kk / 32;
        c = (kk % 32) / 8;
    } else {
        c = kk / 32;
        t = (kk % 32) / 8;
    }
    int64_t tile = (e * NB + nb) * G + g;
    int64_t slot = c * 16 + j;
    int64_t byte = tile * 1024 + slot * 16 + t * 4;
    int64_t bit = 4 * (i / 2) + 16 * (i % 2);
    return byte * 8 + bit;      /* bit offset inside a little-endian word */
}

void oracle_prepack_layout(const uint8_t *w, uint8_t *packed, int64_t E, int64_t K, int64_t N, int is_signed,
                           int layout) {
    memset(packed, 0, (size_t)(E * K * N / 2));
    for (int64_t e = 0; e < E; ++e)
        for (int64_t k = 0; k < K; ++k)
            for (int64_t n = 0; n < N; ++n) {
                int code = nibble(w + e * K * (N / 2), N, k, n);
                if (is_signed) code ^= 0x8;   /* (q + 8) mod 16 for two's complement q */
                int64_t b = packed_bit_index(K, N, e, k, n, layout);
                /* word-relative bit b%32 of the word at byte (b/32)*4: little endian */
                int64_t word_byte = (b / 32) * 4;
                int64_t wb = b % 32;
                packed[word_byte + wb / 8] |= (uint8_t)(code << (wb % 8));
            }
}

void oracle_unpack_layout(const uint8_t *packed, uint8_t *w, int64_t E, int64_t K, int64_t N, int is_signed,
                          int layout) {
    memset(w, 0, (size_t)(E * K * N / 2));
    for (int64_t e = 0; e < E; ++e)
        for (int64_t k = 0; k < K; ++k)
            for (int64_t n = 0; n < N; ++n) {
                int64_t b = packed_bit_index(K, N, e, k, n, layout);
                int64_t word_byte = (b / 32) * 4;
                int64_t wb = b % 32;
                int code = (packed[word_byte + wb / 8] >> (wb % 8)) & 0xF;
                if (is_signed) code ^= 0x8;
                uint8_t *dst = w + e * K * (N / 2) + k * (N / 2) + n / 2;
                *dst |= (uint8_t)((n & 1) ? (code << 4) : code);
            }
}

void oracle_prepack(const uint8_t *w, uint8_t *packed, int64_t E, int64_t K, int64_t N, int is_signed) {
    oracle_prepack_layout(w, packed, E, K, N, is_signed, 0);
}

void oracle_unpack(const uint8_t *packed, uint8_t *w, int64_t E, int64_t K, int64_t N, int is_signed) {
    oracle_unpack_layout(packed, w, E, K, N, is_signed, 0);
}

/* ------------------------------------------------------------------------- */
/* MoE fused-experts chain                                                    */
/* ------------------------------------------------------------------------- */

int64_t oracle_moe_align(const int32_t *topk_ids, int64_t T, int64_t topk, int64_t E,
                         int32_t *offsets, int32_t *sorted, int32_t *row_of) {
    int64_t n = T * topk;
    /* counting sort, stable in the entry index */
    int64_t *next = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
    assert(next);
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_ids[i];
        if (e >= 0 && e < E) next[e + 1] += 1;
    }
    for (int64_t e = 0; e < E; ++e) next[e + 1] += next[e];
    for (int64_t e = 0; e <= E; ++e) offsets[e] = (int32_t)next[e];
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_ids[i];
        if (e >= 0 && e < E) {
            int64_t r = next[e]++;
            sorted[r] = (int32_t)i;
            row_of[i] = (int32_t)r;
        } else {
            row_of[i] = -1;
        }
    }
    int64_t R = offsets[E];
    free(next);
    return R;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

void oracle_silu_and_mul(const uint16_t *h, int64_t R, int64_t I, int dtype, uint16_t *a) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t i = 0; i < I; ++i) {
            double g = to_double(h[r * 2 * I + i], dtype);
            double u = to_double(h[r * 2 * I + I + i], dtype);
            double v = silu(g) * u;
            oracle_round_array(&v, &a[r * I + i], 1, dtype);
        }
}

void oracle_moe_sum(const uint16_t *o, const int32_t *row_of, const float *topk_w,
                    int64_t T, int64_t topk, int64_t N, int dtype, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < topk; ++k) {
                int32_t r = row_of[t * topk + k];
                if (r < 0) continue;
                s += (double)topk_w[t * topk + k] * to_double(o[(int64_t)r * N + n], dtype);
            }
            oracle_round_array(&s, &out[t * N + n], 1, dtype);
        }
}

void oracle_fused_moe(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                      const uint8_t *w13, const uint16_t *s13, const uint8_t *z13,
                      const uint8_t *w2, const uint16_t *s2, const uint8_t *z2,
                      int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I,
                      int64_t group, int dtype, const int64_t *tok, int64_t P, uint16_t *out) {
    (void)T;
    int64_t G1 = H / group, G2 = I / group;
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(2 * I));
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
    uint16_t *ob = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    assert(h && a && ob && acc);
    for (int64_t p = 0; p < P; ++p) {
        int64_t t = tok[p];
        for (int64_t n = 0; n < H; ++n) acc[n] = 0.0;
        for (int64_t k = 0; k < topk; ++k) {
            int32_t e = topk_ids[t * topk + k];
            if (e < 0 || e >= E) continue;
            /* gate/up projection of the token, rounded to the dtype */
            oracle_w4a16(x + t * H, w13 + e * H * I, s13 + e * G1 * 2 * I,
                         z13 ? z13 + e * G1 * I : NULL, 1, H, 2 * I, group, dtype, NULL, h);
            oracle_silu_and_mul(h, 1, I, dtype, a);
            /* down projection, rounded to the dtype */
            oracle_w4a16(a, w2 + e * I * (H / 2), s2 + e * G2 * H, z2 ? z2 + e * G2 * (H / 2) : NULL,
                         1, I, H, group, dtype, NULL, ob);
            for (int64_t n = 0; n < H; ++n) acc[n] += (double)topk_w[t * topk + k] * to_double(ob[n], dtype);
        }
        oracle_round_array(acc, out + p * H, H, dtype);
    }
    free(h); free(a); free(ob); free(acc);
}

/* ------------------------------------------------------------------------- */
/* W4A8-MXFP4 (OCP MX formats)                                                */
/* ------------------------------------------------------------------------- */

double oracle_e4m3_to_double(uint8_t v) {
    int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
    if (e == 15 && m == 7) return NAN;
    double x = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -x : x;
}

double oracle_e2m1_to_double(uint8_t v) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double x = mag[v & 7];
    return (v & 8) ? -x : x;
}

double oracle_e8m0_to_double(uint8_t v) { return v == 255 ? NAN : ldexp(1.0, (int)v - 127); }

/* E4M3 code of a finite double, round to nearest even over the representable
 * values, saturated to +-448.  Written as a search over the 127 non-negative
 * finite codes (monotone in the code), so it is plainly the nearest-value
 * rounding of the definition. */
static uint8_t e4m3_rne_sat(double v) {
    int neg = signbit(v) != 0;
    double a = fabs(v);
    if (a >= 448.0) return (uint8_t)((neg << 7) | 0x7E);
    int best = 0;
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(oracle_e4m3_to_double((uint8_t)c) - a), db = fabs(oracle_e4m3_to_double((uint8_t)best) - a);
        if (d < db || (d == db && (c & 1) == 0 && (best & 1) == 1)) best = c;
    }
    return (uint8_t)((neg << 7) | best);
}

void oracle_mxfp8_quantize(const uint16_t *x, int64_t M, int64_t K, int dtype, uint8_t *qx, uint8_t *sx) {
    int64_t B = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < B; ++b) {
            double amax = 0.0;
            for (int64_t k = 32 * b; k < 32 * b + 32; ++k) {
                double a = fabs(to_double(x[m * K + k], dtype));
                if (a > amax) amax = a;
            }
            int e = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
                e = ex - 1 - 8;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            sx[m * B + b] = (uint8_t)(e + 127);
            for (int64_t k = 32 * b; k < 32 * b + 32; ++k)
                qx[m * K + k] = e4m3_rne_sat(ldexp(to_double(x[m * K + k], dtype), -e));
        }
}

void oracle_w4a8_mxfp4(const uint8_t *qx, const uint8_t *sx, const uint8_t *w, const uint8_t *sw,
                       int64_t M, int64_t K, int64_t N, int dtype, double *y64, uint16_t *y) {
    if (M <= 0) return;
    int64_t B = K / 32;
    /* Step 1: both operands decoded once into fp64 (exact: an E4M3 or E2M1
     * value times a power of two).  a[m][k] = E4M3(qx) * 2^(sx - 127) for the
     * 32-block k / 32 of row m; b[k][n] = E2M1(code of (k, n)) * 2^(sw - 127)
     * for the 32-block k / 32 of column n; the low nibble is the even column. */
    double *a = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    double *b = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    assert(a && b);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            a[m * K + k] = oracle_e4m3_to_double(qx[m * K + k]) * oracle_e8m0_to_double(sx[m * B + k / 32]);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            uint8_t byte = w[k * (N / 2) + n / 2];
            uint8_t code = (n & 1) ? (byte >> 4) : (byte & 0xF);
            b[k * N + n] = oracle_e2m1_to_double(code) * oracle_e8m0_to_double(sw[(k / 32) * N + n]);
        }
    double *acc = y64 ? y64 : (double *)malloc(sizeof(double) * (size_t)(M * N));
    assert(acc);
    /* Step 2: acc[m][n] = sum_k a[m][k] * b[k][n], each sum in ascending k
     * (every product is exact in fp64; the loop over n only runs independent
     * sums side by side). */
    const int64_t NC = 512;
    int64_t nchunks = (N + NC - 1) / NC;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n0 = c * NC, n1 = n0 + NC < N ? n0 + NC : N;
            double *row = acc + m * N;
            for (int64_t n = n0; n < n1; ++n) row[n] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double av = a[m * K + k];
                const double *br = b + k * N;
                for (int64_t n = n0; n < n1; ++n) row[n] += av * br[n];
            }
        }
    /* Step 3: one rounding to the output dtype. */
    if (y) oracle_round_array(acc, y, M * N, dtype);
    if (!y64) free(acc);
    free(a);
    free(b);
}

/* ------------------------------------------------------------------------- */
/* W8A16                                                                      */
/* ------------------------------------------------------------------------- */

void oracle_w8a16(const uint16_t *x, const uint8_t *w, const uint16_t *scale, const uint8_t *zero,
                  int64_t M, int64_t K, int64_t N, int64_t group, int dtype, double *y64, uint16_t *y) {
    if (M <= 0) return;
    /* dequant(W)[k][n] = (q - z) * s: |q - z| < 2^9 and s has at most 11
     * significant bits, so every value is exact in fp64 */
    double *wd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    assert(wd);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const int64_t g = k / group;
            const uint8_t b = w[k * N + n];
            const int q = zero ? (int)b : (int)(int8_t)b;
            const int z = zero ? (int)zero[g * N + n] : 0;
            wd[k * N + n] = (double)(q - z) * to_double(scale[g * N + n], dtype);
        }
    double *acc = y64 ? y64 : (double *)malloc(sizeof(double) * (size_t)M * (size_t)N);
    assert(acc);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *row = acc + m * N;
        for (int64_t n = 0; n < N; ++n) row[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xv = to_double(x[m * K + k], dtype);
            const double *wr = wd + k * N;
            for (int64_t n = 0; n < N; ++n) row[n] += xv * wr[n];
        }
    }
    if (y) oracle_round_array(acc, y, M * N, dtype);
    if (!y64) free(acc);
    free(wd);
}

/* ------------------------------------------------------------------------- */
/* W4A16 with floating-point zero points                                      */
/* ------------------------------------------------------------------------- */

void oracle_w4a16_fzero(const uint16_t *x, const uint8_t *w, const uint16_t *scale, const uint16_t *zf,
                        int64_t M, int64_t K, int64_t N, int64_t group, int dtype, double *y64, uint16_t *y) {
    if (M <= 0) return;
    /* (u - zf) * s: u < 16, zf and s 16-bit floats, so every value is exact in fp64 */
    double *wd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    assert(wd);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const int64_t g = k / group;
            const int u = nibble(w, N, k, n);
            wd[k * N + n] = ((double)u - to_double(zf[g * N + n], dtype)) * to_double(scale[g * N + n], dtype);
        }
    double *acc = y64 ? y64 : (double *)malloc(sizeof(double) * (size_t)M * (size_t)N);
    assert(acc);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *row = acc + m * N;
        for (int64_t n = 0; n < N; ++n) row[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xv = to_double(x[m * K + k], dtype);
            const double *wr = wd + k * N;
            for (int64_t n = 0; n < N; ++n) row[n] += xv * wr[n];
        }
    }
    if (y) oracle_round_array(acc, y, M * N, dtype);
    if (!y64) free(acc);
    free(wd);
}

void oracle_w8a16_fzero(const uint16_t *x, const uint8_t *w, const uint16_t *scale, const uint16_t *zf,
                        int64_t M, int64_t K, int64_t N, int64_t group, int dtype, double *y64, uint16_t *y) {
    if (M <= 0) return;
    double *wd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    assert(wd);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const int64_t g = k / group;
            wd[k * N + n] = ((double)w[k * N + n] - to_double(zf[g * N + n], dtype)) * to_double(scale[g * N + n], dtype);
        }
    double *acc = y64 ? y64 : (double *)malloc(sizeof(double) * (size_t)M * (size_t)N);
    assert(acc);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *row = acc + m * N;
        for (int64_t n = 0; n < N; ++n) row[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xv = to_double(x[m * K + k], dtype);
            const double *wr = wd + k * N;
            for (int64_t n = 0; n < N; ++n) row[n] += xv * wr[n];
        }
    }
    if (y) oracle_round_array(acc, y, M * N, dtype);
    if (!y64) free(acc);
    free(wd);
}
