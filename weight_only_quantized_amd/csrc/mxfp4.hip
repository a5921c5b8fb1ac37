// mxfp4.hip — W4A8-MXFP4: MXFP4 weights (E2M1 codes with one E8M0 scale per
// 32 K rows and column) times MXFP8 activations (E4M3 codes with one E8M0
// scale per row and 32 K elements), formats as in the OCP Microscaling (MX)
// v1.0 specification; the path itself is the Humming article's W4A8-MXFP4
// route.  The article converts MXFP4 weights inside the kernel because the
// GPUs it targets have no MXFP4 matrix cores; gfx950 has them: the
// block-scaled instruction v_mfma_scale_f32_16x16x128_f8f6f4 takes E4M3 A,
// E2M1 B and both E8M0 scales directly, so the weights go from memory into
// the matrix core untouched and no vector-ALU dequantization is left.
//
// Operand layout of that instruction (16 x 16 x 128, fp8 A, fp4 B):
//   A (8 registers): lane l feeds row l % 16; with h = l / 16, bytes 0..15
//     hold k = 16h + i and bytes 16..31 hold k = 64 + 16h + i (i = 0..15);
//   B (4 registers): lane l feeds column l % 16 and rows k = 32h + r,
//     r = 0..31, as nibble r of its 16 bytes (low nibble first);
//   scales: lane l's A scale belongs to row l % 16, k-block h (32 rows); its B
//     scale to column l % 16, k-block h (E8M0 in the low byte);
//   D: register r of lane l is row 4h + r, column l % 16.
//
// Prepacked weight tile (1088 bytes per 16-column block and 128-row group):
// bytes 0..1023 are the 64 lanes' B operands (16 bytes each, lane-major), bytes
// 1024..1087 the 64 lanes' B scales.  One 128-bit and one 8-bit load per lane
// deliver a whole instruction's weight operand.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int kMxTileBytes = 1088;
constexpr int kMxCodeBytes = 1024;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_mx(const i32x8_t &a, const i32x8_t &b, const f32x4_t &c, int sa, int sb) {
    // cbsz = 0: A is E4M3; blgp = 4: B is E2M1 (only the low 4 registers read)
    f32x4_t r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
    keep_live(r, a, b);
    return r;
}

// Shared exponent of an MXFP8 block (OCP MX: floor(log2 max|x|) minus the
// largest E4M3 exponent, 8), clamped to the E8M0 range.  For a zero or
// subnormal maximum the exponent field gives -127 and the clamp the smallest
// scale, which is what the exact floor(log2) would give as well.
__device__ __forceinline__ int mx_shared_exp(float amax) {
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values scaled by 2^-e (exact), clamped to the largest E4M3 magnitude
// and converted with round-to-nearest-even, packed into one word (byte i =
// value i).
__device__ __forceinline__ uint32_t mx_e4m3x4(float a, float b, float c, float d, int e) {
    a = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(a, -e), -448.f, 448.f);
    b = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(b, -e), -448.f, 448.f);
    c = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(c, -e), -448.f, 448.f);
    d = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(d, -e), -448.f, 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Eight 16-bit values (one 128-bit load) as fp32.
template <int DT>
__device__ __forceinline__ void unpack8(const u32x4_t &v, float (&f)[8]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t w = v[t];
        f[2 * t] = h2f<DT>((uint16_t)(w & 0xFFFFu));
        f[2 * t + 1] = h2f<DT>((uint16_t)(w >> 16));
    }
}

__device__ __forceinline__ float amax8(const float (&f)[8]) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

// ---------------------------------------------------------------------------
// Weight prepack: w[E][K][N/2] E2M1 codes (low nibble = even column) and
// sw[E][K/32][N] E8M0 scales into 1088-byte tiles ordered (expert, 16-column
// block, 128-row group).  One 64-thread workgroup per tile.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) mx_prepack_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ sw,
                                                        uint8_t *__restrict__ out, int64_t K, int64_t N) {
    const int64_t G = K / kGroup, NB = N / 16;
    const int64_t tile = blockIdx.x;                 // (e * NB + nb) * G + g
    const int64_t g = tile % G;
    const int64_t nb = (tile / G) % NB;
    const int64_t e = tile / (G * NB);
    const int L = threadIdx.x;

    __shared__ uint64_t rows[kGroup];                 // 16 codes of each row
    const uint8_t *src = w + e * K * (N / 2) + (g * kGroup) * (N / 2) + nb * 8;
    for (int r = L; r < kGroup; r += 64) rows[r] = *reinterpret_cast<const uint64_t *>(src + (int64_t)r * (N / 2));
    __syncthreads();

    const int h = L >> 4, j = L & 15;
    u32x4_t slot;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= ((uint32_t)(rows[32 * h + 8 * t + i] >> (4 * j)) & 0xFu) << (4 * i);
        slot[t] = word;
    }
    uint8_t *dst = out + tile * kMxTileBytes;
    *reinterpret_cast<u32x4_t *>(dst + L * 16) = slot;
    dst[kMxCodeBytes + L] = sw[e * (K / 32) * N + (4 * g + h) * N + nb * 16 + j];
}

// ---------------------------------------------------------------------------
// MXFP8 quantization of activations: x[M][K] -> qx[M][K] E4M3 codes and
// sx[M][K/32] E8M0 scales.  Four consecutive lanes own one 32-element block
// (8 elements each, one 128-bit load) and agree on its maximum with two
// cross-lane exchanges.
// ---------------------------------------------------------------------------
template <int DT>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const uint16_t *__restrict__ x, uint8_t *__restrict__ qx,
                                                          uint8_t *__restrict__ sx, int64_t n8) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // n8 is a multiple of 4 and quads are lane-aligned: a quad is all in or all out
    if (t >= n8) return;
    float f[8];
    unpack8<DT>(ld128(x + t * 8), f);
    float m = amax8(f);
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int e = mx_shared_exp(m);
    u32x2_t q;
    q[0] = mx_e4m3x4(f[0], f[1], f[2], f[3], e);
    q[1] = mx_e4m3x4(f[4], f[5], f[6], f[7], e);
    *reinterpret_cast<u32x2_t *>(qx + t * 8) = q;
    if ((t & 3) == 0) sx[t >> 2] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------------------
// Small-M GEMM: split-K over the waves of a workgroup, reduced through LDS
// (the structure of the W4A16 decode kernel).  A workgroup owns NB 16-column
// blocks and a 16-row chunk of the output (blockIdx.y); wave w owns the SG
// 128-row groups w*SG .. w*SG+SG-1 for all NB blocks.
//
// FUSED: the wave reads its slice of the 16-bit activations and quantizes it
// to MXFP8 in registers, straight into the A operand: lane l holds for row
// l % 16 the 16 elements k = 16h + i (block h/2 of the group) and the 16
// elements 64 + 16h + i (block 2 + h/2); its partner lane l ^ 16 holds the
// other halves of the same two blocks, so one exchange gives both block
// maxima.  Lane l's A scale (block h) then sits in lane 32*(h & 1) + l % 16,
// low half for h < 2, high half otherwise.  Every workgroup repeats this for
// its slice (a few hundred vector instructions per wave, from L2), which
// saves the separate quantization launch.
// Otherwise (prequantized) the A operand is two 128-bit loads of qx and one
// byte of sx per group.
//
// Per weight tile a wave then issues one 128-bit and one 8-bit buffer load and
// one block-scaled matrix-core instruction, chained on the block's
// accumulator across groups (the scales are applied inside the instruction).
// ---------------------------------------------------------------------------
constexpr int kMxSmallMaxWaves = 16;

template <int DT, bool FUSED, int NB, int SG, int D>
__global__ void __launch_bounds__(kMxSmallMaxWaves * 64)
mx_small_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ qx, const uint8_t *__restrict__ sx,
                const uint8_t *__restrict__ wp, uint16_t *__restrict__ y, int M, int64_t K, int64_t N) {
    static_assert(NB * SG <= 16, "tile pipeline fits in registers");
    constexpr int T = NB * SG;
    const int G = (int)(K / kGroup);
    const int W = blockDim.x >> 6;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;
    const int h = lane >> 4;
    const int64_t nb0 = (int64_t)blockIdx.x * NB;
    const int m0 = blockIdx.y * 16;
    const int g0 = wave * SG;

    // rows past M read row M - 1 (finite, in bounds); their results are dropped
    const int64_t row = m0 + j < M ? m0 + j : M - 1;

    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wp + nb0 * G * kMxTileBytes), (short)0, NB * G * kMxTileBytes, 0x00020000);
    u32x4_t raw[T];
    int sb[T];
    auto issue = [&](int q) {
        const int b = q / SG, i = q % SG;
        const int g = g0 + i < G ? g0 + i : G - 1;
        const int toff = (b * G + g) * kMxTileBytes;
        raw[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, lane * 16, toff, 0));
        sb[q] = __builtin_amdgcn_raw_buffer_load_b8(wrsrc, kMxCodeBytes + lane, toff, 0);
    };
    // the first D weight tiles go out before the activation slice is read
    // and quantized, so the two memory latencies overlap
#pragma unroll
    for (int q = 0; q < D && q < T; ++q) issue(q);
    __builtin_amdgcn_sched_barrier(0);

    i32x8_t a[SG];
    int sa[SG];
#pragma unroll
    for (int i = 0; i < SG; ++i) {
        const bool live = g0 + i < G;
        const int64_t g = live ? g0 + i : G - 1;
        if constexpr (FUSED) {
            const uint16_t *xb = x + row * K + g * kGroup + 16 * h;
            float lo0[8], lo1[8], hi0[8], hi1[8];
            unpack8<DT>(ld128(xb), lo0);
            unpack8<DT>(ld128(xb + 8), lo1);
            unpack8<DT>(ld128(xb + 64), hi0);
            unpack8<DT>(ld128(xb + 72), hi1);
            float mlo = fmaxf(amax8(lo0), amax8(lo1));
            float mhi = fmaxf(amax8(hi0), amax8(hi1));
            mlo = fmaxf(mlo, __shfl_xor(mlo, 16));
            mhi = fmaxf(mhi, __shfl_xor(mhi, 16));
            const int elo = mx_shared_exp(mlo), ehi = mx_shared_exp(mhi);
            a[i][0] = (int)mx_e4m3x4(lo0[0], lo0[1], lo0[2], lo0[3], elo);
            a[i][1] = (int)mx_e4m3x4(lo0[4], lo0[5], lo0[6], lo0[7], elo);
            a[i][2] = (int)mx_e4m3x4(lo1[0], lo1[1], lo1[2], lo1[3], elo);
            a[i][3] = (int)mx_e4m3x4(lo1[4], lo1[5], lo1[6], lo1[7], elo);
            a[i][4] = (int)mx_e4m3x4(hi0[0], hi0[1], hi0[2], hi0[3], ehi);
            a[i][5] = (int)mx_e4m3x4(hi0[4], hi0[5], hi0[6], hi0[7], ehi);
            a[i][6] = (int)mx_e4m3x4(hi1[0], hi1[1], hi1[2], hi1[3], ehi);
            a[i][7] = (int)mx_e4m3x4(hi1[4], hi1[5], hi1[6], hi1[7], ehi);
            const int packed = (elo + 127) | (ehi + 127) << 8;
            const int v = __builtin_amdgcn_ds_bpermute((32 * (h & 1) + j) << 2, packed);
            sa[i] = (v >> (8 * (h >> 1))) & 0xFF;
        } else {
            const uint8_t *qb = qx + row * K + g * kGroup + 16 * h;
            const u32x4_t q0 = ld128(qb), q1 = ld128(qb + 64);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a[i][t] = (int)q0[t];
                a[i][4 + t] = (int)q1[t];
            }
            sa[i] = sx[row * (K / 32) + 4 * g + h];
        }
        // a group past the end of K (G not a multiple of SG) contributes zero
        if (!live) a[i] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }

    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < T; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        if (q + D < T) issue(q + D);
        __builtin_amdgcn_sched_barrier(0);
        const int b = q / SG, i = q % SG;
        const i32x8_t bv = {(int)raw[q][0], (int)raw[q][1], (int)raw[q][2], (int)raw[q][3], 0, 0, 0, 0};
        acc[b] = mfma_mx(a[i], bv, acc[b], sa[i], sb[q]);
    }

    __shared__ float red[kMxSmallMaxWaves][NB][16][17];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][b][4 * h + r][j] = acc[b][r];
    __syncthreads();

    for (int idx = threadIdx.x; idx < NB * 256; idx += W * 64) {
        const int b = idx >> 8, r = (idx >> 4) & 15, col = idx & 15;
        if (m0 + r < M) {
            float sum = 0.f;
            for (int w = 0; w < W; ++w) sum += red[w][b][r][col];
            y[(int64_t)(m0 + r) * N + (nb0 + b) * 16 + col] = f2h<DT>(sum);
        }
    }
}

// ---------------------------------------------------------------------------
// Large-M GEMM from prequantized activations.  Workgroup tile BM x BN over
// the whole K range; WM x WN waves, each owning a TM x TN sub-tile of
// (TM/16) x (TN/16) block-scaled 16x16x128 instructions per 128-row group.
//  * A (E4M3 codes and their E8M0 scales): the BM x 128 slice of one group
//    is staged in LDS, double-buffered; the next group's slice is fetched into
//    registers while the current one is multiplied and written to the other
//    buffer halfway through the products.  An LDS row holds the 128 code bytes
//    and the row's 4 scale bytes in a 144-byte stride, so the 128-bit operand
//    reads of 8 consecutive rows fall in disjoint banks.
//  * B: every wave loads its own tiles (one 128-bit and one 8-bit load per
//    lane per 16 columns) straight from memory into the operand registers,
//    the next group's set in flight while the current one is used.
//  * The scales are applied inside the instruction, so each accumulator
//    chains across all groups and is rounded once at the end.
// ---------------------------------------------------------------------------
constexpr int kMxRowB = 144;

// XCDs of an MI355X; workgroups are dispatched to them round-robin.
constexpr int kMxXcds = 8;

// GROUPED (MoE): rows offsets[e] .. offsets[e+1]-1 are multiplied by expert
// e's weights; the work items (row tile, column block) are numbered on the
// device from the offsets (prefix sum of ceil(rows_e / BM)), and XCD x takes
// an equal contiguous range of them, so an expert's row tiles and weights
// stay in one L2.  Surplus workgroups exit at once.
template <int DT, int BM, int BN, int WM, int WN, bool GROUPED>
__global__ void __launch_bounds__(WM * WN * 64, 2)
mx_tile_kernel(const uint8_t *__restrict__ qx, const uint8_t *__restrict__ sx, const int32_t *__restrict__ offsets,
               const uint8_t *__restrict__ wp, uint16_t *__restrict__ y, int64_t M, int64_t K, int64_t N, int E) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int RT = TM / 16, CT = TN / 16;
    constexpr int XP = BM * 8 / NT;                  // 16-byte code chunks per thread and group
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert((BM * 8) % NT == 0 && BM <= NT, "A staging must divide evenly");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BM * kMxRowB];

    // the wave index is uniform: readfirstlane lets the compiler keep every
    // value derived from it (the weight-tile offsets) in scalar registers, as
    // the buffer loads' scalar offset operand requires
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int j = lane & 15, h = lane >> 4;
    const int G = (int)(K / kGroup);
    int64_t row0, row_end, n0, e = 0;
    if constexpr (GROUPED) {
        __shared__ int s_info[5];      // expert, row tile within it, total row tiles, the expert's offsets
        __shared__ int scan[NT];
        // row tiles of expert ee (0 past E); o0, o1 get its offsets
        auto tiles_of = [&](int ee, int &o0, int &o1) {
            o0 = ee < E ? offsets[ee] : 0;
            o1 = ee < E ? offsets[ee + 1] : 0;
            const int cnt = o1 - o0;
            return cnt > 0 ? (cnt + BM - 1) / BM : 0;
        };
        // this workgroup's item: slot bid / 8 of XCD bid % 8's contiguous range
        const int64_t ncb = (N + BN - 1) / BN;
        const int64_t bid = blockIdx.x, xcd = bid % kMxXcds;
        int64_t item;
        if (E <= 64) {
            // one wave: inclusive scan of the experts' row tiles over its
            // lanes, then the expert holding this item's row tile
            if (wave == 0) {
                int o0, o1;
                const int tl = tiles_of(lane, o0, o1);
                const int incl = wave_incl_scan(tl);
                const int64_t total = __builtin_amdgcn_readlane(incl, 63);
                const int64_t items = total * ncb;
                const int64_t it = items * xcd / kMxXcds + bid / kMxXcds;
                const int tile = (int)(it / ncb);
                if (lane == 0) {
                    s_info[0] = -1;
                    s_info[2] = (int)total;
                }
                if (it < items * (xcd + 1) / kMxXcds && lane < E && tile >= incl - tl && tile < incl) {
                    s_info[0] = lane;
                    s_info[1] = tile - (incl - tl);
                    s_info[3] = o0;
                    s_info[4] = o1;
                }
            }
            __syncthreads();
            // values read back from LDS are the same in every lane:
            // readfirstlane keeps them (and the tile offsets derived from
            // them) scalar
            const int64_t items = (int64_t)__builtin_amdgcn_readfirstlane(s_info[2]) * ncb;
            item = items * xcd / kMxXcds + bid / kMxXcds;
            if (item >= items * (xcd + 1) / kMxXcds) return;   // uniform: surplus workgroup
        } else {
        if (tid == 0) {
            s_info[0] = -1;
            s_info[2] = 0;
        }
        __syncthreads();
        int part = 0;
        for (int ee = tid; ee < E; ee += NT) {
            int o0, o1;
            part += tiles_of(ee, o0, o1);
        }
        part = __builtin_amdgcn_readlane(wave_incl_scan(part), 63);
        if (lane == 0) atomicAdd(&s_info[2], part);
        __syncthreads();
        const int64_t items = (int64_t)__builtin_amdgcn_readfirstlane(s_info[2]) * ncb;
        item = items * xcd / kMxXcds + bid / kMxXcds;
        if (item >= items * (xcd + 1) / kMxXcds) return;   // uniform: surplus workgroup
        const int tile = (int)(item / ncb);
        int carry = 0;
        for (int base = 0; base < E; base += NT) {
            const int ee = base + tid;
            int o0, o1;
            const int tl = tiles_of(ee, o0, o1);
            scan[tid] = tl;
            __syncthreads();
            for (int off = 1; off < NT; off <<= 1) {
                const int v = tid >= off ? scan[tid - off] : 0;
                __syncthreads();
                scan[tid] += v;
                __syncthreads();
            }
            const int incl = scan[tid] + carry, excl = incl - tl;
            if (ee < E && tile >= excl && tile < incl) {
                s_info[0] = ee;
                s_info[1] = tile - excl;
                s_info[3] = o0;
                s_info[4] = o1;
            }
            carry += scan[NT - 1];
            __syncthreads();
        }
        }
        n0 = (item % ncb) * BN;
        e = __builtin_amdgcn_readfirstlane(s_info[0]);   // always found: tile < total row tiles
        // the expert's offsets as its scan lane read them (no second load)
        const int64_t oe = __builtin_amdgcn_readfirstlane(s_info[3]), oe1 = __builtin_amdgcn_readfirstlane(s_info[4]);
        row0 = oe + (int64_t)__builtin_amdgcn_readfirstlane(s_info[1]) * BM;
        row_end = oe1 < M ? oe1 : M;   // offsets[E] == R by contract
    } else {
        row0 = (int64_t)blockIdx.x * BM;
        row_end = M;
        n0 = (int64_t)blockIdx.y * BN;
    }
    // a wave whose columns lie past N (N % 64 == 0: all in or all out) runs
    // the loop on the last columns with every load in bounds and stores nothing
    const bool wave_cols = n0 + (int64_t)wn * TN < N;
    const int64_t wcol0 = wave_cols ? n0 + (int64_t)wn * TN : N - TN;
    wp += e * (N / 16) * (int64_t)G * kMxTileBytes;

    // ---- A staging: rows past the tile's end read its last row (never stored)
    u32x4_t ar[XP];
    const uint8_t *arow[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int id = p * NT + tid, r = id >> 3, c = id & 7;
        const int64_t grow = row0 + r < row_end ? row0 + r : row_end - 1;
        arow[p] = qx + grow * K + c * 16;
    }
    const int64_t srow = row0 + tid < row_end ? row0 + tid : row_end - 1;
    const uint8_t *sxrow = sx + srow * (K / 32);
    uint32_t asc = 0;
    auto load_a = [&](int g) {
#pragma unroll
        for (int p = 0; p < XP; ++p) ar[p] = ld128(arow[p] + (int64_t)g * kGroup);
        if (tid < BM) asc = *reinterpret_cast<const uint32_t *>(sxrow + 4 * g);
    };
    auto store_a = [&](int buf) {
        uint8_t *base = lds + buf * BM * kMxRowB;
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int id = p * NT + tid, r = id >> 3, c = id & 7;
            *reinterpret_cast<u32x4_t *>(base + r * kMxRowB + c * 16) = ar[p];
        }
        if (tid < BM) *reinterpret_cast<uint32_t *>(base + tid * kMxRowB + 128) = asc;
    };

    // ---- B: byte offset of this lane's slot in each column block's group 0 ---
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wp), (short)0, 0x7FFFFFFF, 0x00020000);
    int boff[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) boff[ct] = (int)(((wcol0 >> 4) + ct) * G * kMxTileBytes);
    u32x4_t bq[CT], bn[CT];
    int bs[CT], bsn[CT];
    auto load_b = [&](int g, u32x4_t (&dst)[CT], int (&sdst)[CT]) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int toff = boff[ct] + g * kMxTileBytes;
            dst[ct] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, lane * 16, toff, 0));
            sdst[ct] = __builtin_amdgcn_raw_buffer_load_b8(wrsrc, kMxCodeBytes + lane, toff, 0);
        }
    };

    f32x4_t acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_b(0, bq, bs);
    store_a(0);
    __syncthreads();

    const int arow0 = wm * TM + j;
    auto step = [&](int g, const u32x4_t (&bw)[CT], const int (&sw)[CT], u32x4_t (&bnx)[CT], int (&snx)[CT]) {
        const int buf = g & 1;
        const int gn = g + 1 < G ? g + 1 : g;     // the last step re-reads: no branch around loads
        load_a(gn);
        load_b(gn, bnx, snx);
        const uint8_t *abase = lds + buf * BM * kMxRowB + arow0 * kMxRowB;
        // A operands are read from LDS one 16-row block ahead of their use
        auto read_a = [&](int rt, i32x8_t &av, int &sa) {
            const uint8_t *ap = abase + rt * 16 * kMxRowB;
            const u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(ap + 16 * h);
            const u32x4_t a1 = *reinterpret_cast<const u32x4_t *>(ap + 64 + 16 * h);
            sa = ap[128 + h];
            av = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        };
        i32x8_t avs[2];
        int sas[2];
        read_a(0, avs[0], sas[0]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            // the scheduling barriers keep the next block's LDS reads ahead of
            // this block's products (left alone, the compiler issues them after
            // the products and waits at once, draining the matrix pipe)
            if (rt + 1 < RT) read_a(rt + 1, avs[(rt + 1) & 1], sas[(rt + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            const i32x8_t &av = avs[rt & 1];
            const int sa = sas[rt & 1];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                // an fp4 B operand occupies the low four registers only
                const u32x4_t b4 = bw[ct];
                const i32x8_t bv = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(b4, b4, 0, 1, 2, 3, -1, -1, -1, -1));
                acc[rt][ct] = mfma_mx(av, bv, acc[rt][ct], sa, sw[ct]);
            }
            __builtin_amdgcn_sched_barrier(0);
            // stage the next slice halfway through the products; the buffer
            // written was last read in the previous step, before its barrier
            if (rt == RT / 2) store_a(buf ^ 1);
        }
        if (RT == 1) store_a(buf ^ 1);
        __syncthreads();
    };
    for (int g = 0; g < G; g += 2) {
        step(g, bq, bs, bn, bsn);
        if (g + 1 < G) step(g + 1, bn, bsn, bq, bs);
    }

    if (!wave_cols) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t col = wcol0 + ct * 16 + j;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = row0 + wm * TM + rt * 16 + 4 * h + r;
                if (row < row_end) y[row * N + col] = f2h<DT>(acc[rt][ct][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
size_t mx_prepacked_bytes(int64_t E, int64_t K, int64_t N) {
    return (size_t)E * (size_t)(K / kGroup) * (size_t)(N / 16) * kMxTileBytes;
}

hipError_t launch_mx_prepack(const void *w, const void *sw, void *out, int64_t E, int64_t K, int64_t N,
                             hipStream_t stream) {
    const int64_t tiles = E * (K / kGroup) * (N / 16);
    for (int64_t e = 0; e < E; ++e) {
        // one launch per expert keeps the grid within 2^31 workgroups for any size
        const int64_t per = tiles / E;
        hipLaunchKernelGGL(mx_prepack_kernel, dim3((unsigned)per), dim3(64), 0, stream,
                           (const uint8_t *)w + e * K * (N / 2), (const uint8_t *)sw + e * (K / 32) * N,
                           (uint8_t *)out + e * per * kMxTileBytes, K, N);
    }
    return hipGetLastError();
}

hipError_t launch_mx_quantize(const void *x, void *qx, void *sx, int64_t M, int64_t K, int dt, hipStream_t stream) {
    const int64_t n8 = M * K / 8;
    if (n8 == 0) return hipSuccess;
    const dim3 grid((unsigned)((n8 + 255) / 256));
    if (dt == DT_BF16)
        hipLaunchKernelGGL(mx_quantize_kernel<DT_BF16>, grid, dim3(256), 0, stream, (const uint16_t *)x,
                           (uint8_t *)qx, (uint8_t *)sx, n8);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<DT_F16>, grid, dim3(256), 0, stream, (const uint16_t *)x,
                           (uint8_t *)qx, (uint8_t *)sx, n8);
    return hipGetLastError();
}

// Small-kernel variants (NB, SG, D); index 0 is the default.
struct MxSmallCfg { int nb, sg, d; };
static constexpr MxSmallCfg kMxSmallCfgs[] = {{4, 2, 4}, {4, 2, 8}, {2, 2, 4}, {4, 1, 4}, {2, 4, 8}, {1, 2, 2}};
static std::atomic<int> g_mx_small_cfg{-1};

int mx_small_config_count() { return (int)(sizeof(kMxSmallCfgs) / sizeof(kMxSmallCfgs[0])); }
void set_mx_small_config(int idx) { g_mx_small_cfg.store(idx, std::memory_order_relaxed); }
int64_t mx_small_max_k() { return (int64_t)kMxSmallMaxWaves * 4 * kGroup; }

template <int DT, bool FUSED, int NB, int SG, int D>
static hipError_t mx_small_launch(const void *x, const void *qx, const void *sx, const void *wp, void *y, int64_t M,
                                  int64_t K, int64_t N, hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t waves = (G + SG - 1) / SG;
    const dim3 grid((unsigned)(N / (16 * NB)), (unsigned)((M + 15) / 16));
    hipLaunchKernelGGL((mx_small_kernel<DT, FUSED, NB, SG, D>), grid, dim3((unsigned)(waves * 64)), 0, stream,
                       (const uint16_t *)x, (const uint8_t *)qx, (const uint8_t *)sx, (const uint8_t *)wp,
                       (uint16_t *)y, (int)M, K, N);
    return hipGetLastError();
}

template <int DT, bool FUSED>
static hipError_t mx_small_dispatch(const void *x, const void *qx, const void *sx, const void *wp, void *y,
                                    int64_t M, int64_t K, int64_t N, hipStream_t stream) {
    const int64_t G = K / kGroup;
    int idx = g_mx_small_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= mx_small_config_count()) idx = 0;
    MxSmallCfg c = kMxSmallCfgs[idx];
    while ((G + c.sg - 1) / c.sg > kMxSmallMaxWaves && c.sg < 4) c.sg *= 2;
    if ((G + c.sg - 1) / c.sg > kMxSmallMaxWaves) return hipErrorInvalidValue;   // K > mx_small_max_k()
    while (c.nb * c.sg > 16) c.nb /= 2;
    if (c.d > c.nb * c.sg) c.d = c.nb * c.sg;
    while ((N / 16) % c.nb != 0) c.nb /= 2;
#define W4_MX(NBV, SGV, DV)                                                                                   \
    if (c.nb == NBV && c.sg == SGV && c.d == DV)                                                              \
        return mx_small_launch<DT, FUSED, NBV, SGV, DV>(x, qx, sx, wp, y, M, K, N, stream);
    W4_MX(4, 2, 8) W4_MX(4, 2, 4) W4_MX(2, 2, 4) W4_MX(4, 1, 4) W4_MX(2, 4, 8) W4_MX(1, 2, 2)
    W4_MX(4, 4, 8) W4_MX(2, 2, 2) W4_MX(1, 4, 4) W4_MX(2, 1, 2) W4_MX(1, 1, 1) W4_MX(1, 2, 1)
    W4_MX(2, 1, 1) W4_MX(4, 1, 2) W4_MX(1, 4, 2) W4_MX(2, 4, 4) W4_MX(4, 2, 2) W4_MX(4, 4, 4)
    W4_MX(4, 1, 1) W4_MX(2, 2, 1) W4_MX(1, 4, 1) W4_MX(2, 4, 2) W4_MX(1, 2, 4)
#undef W4_MX
    return hipErrorInvalidValue;
}

hipError_t launch_mx_gemm_small(const void *x, const void *qx, const void *sx, const void *wp, void *y, int64_t M,
                                int64_t K, int64_t N, int dt, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const bool fused = x != nullptr;
    if (dt == DT_BF16)
        return fused ? mx_small_dispatch<DT_BF16, true>(x, qx, sx, wp, y, M, K, N, stream)
                     : mx_small_dispatch<DT_BF16, false>(x, qx, sx, wp, y, M, K, N, stream);
    return fused ? mx_small_dispatch<DT_F16, true>(x, qx, sx, wp, y, M, K, N, stream)
                 : mx_small_dispatch<DT_F16, false>(x, qx, sx, wp, y, M, K, N, stream);
}


// Tile-kernel variants (BM, BN, WM, WN).  The default follows the workgroup
// count (measured over M = 17..4096 at K = 4096, N = 4096 and 14336): the
// smallest tiles that still give at most 512 workgroups, in the order 32 x 256
// (index 5), 64 x 256 (index 4), 128 x 512 with eight 128 x 64-column waves
// (index 7, the fewest bytes per product), else 128 x 256 with four such waves
// (index 0).  Larger tiles at small M leave most compute units idle (M = 128,
// N = 14336: 24.6 us for index 5 against 53.5 us for index 7); on 4096^3
// index 7 takes 64-77 us against 68-81 us for index 0.
struct MxTileCfg { int bm, bn, wm, wn; };
static constexpr MxTileCfg kMxTileCfgs[] = {{128, 256, 1, 4}, {128, 256, 2, 4}, {128, 128, 2, 2}, {64, 128, 1, 2},
                                            {64, 256, 1, 4}, {32, 256, 1, 4}, {256, 256, 2, 4}, {128, 512, 1, 8}};
static std::atomic<int> g_mx_tile_cfg{-1};

int mx_tile_config_count() { return (int)(sizeof(kMxTileCfgs) / sizeof(kMxTileCfgs[0])); }
void set_mx_tile_config(int idx) { g_mx_tile_cfg.store(idx, std::memory_order_relaxed); }

template <int DT, int BM, int BN, int WM, int WN>
static hipError_t mx_tile_launch(const void *qx, const void *sx, const int32_t *offsets, const void *wp, void *y,
                                 int64_t M, int64_t K, int64_t N, int64_t E, hipStream_t stream) {
    if (offsets) {
        // every expert may end in a partial row tile, hence + E; the items go
        // on a 1-D grid rounded up to whole rounds over the XCDs
        const int64_t ncb = (N + BN - 1) / BN;
        const int64_t slots = (((M + BM - 1) / BM + E) * ncb + kMxXcds - 1) / kMxXcds * kMxXcds;
        if (slots > INT32_MAX) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((mx_tile_kernel<DT, BM, BN, WM, WN, true>), dim3((unsigned)slots), dim3(WM * WN * 64), 0,
                           stream, (const uint8_t *)qx, (const uint8_t *)sx, offsets, (const uint8_t *)wp,
                           (uint16_t *)y, M, K, N, (int)E);
    } else {
        const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
        hipLaunchKernelGGL((mx_tile_kernel<DT, BM, BN, WM, WN, false>), grid, dim3(WM * WN * 64), 0, stream,
                           (const uint8_t *)qx, (const uint8_t *)sx, nullptr, (const uint8_t *)wp, (uint16_t *)y, M,
                           K, N, 1);
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t mx_tile_dispatch(const void *qx, const void *sx, const int32_t *offsets, const void *wp, void *y,
                                   int64_t M, int64_t K, int64_t N, int64_t E, hipStream_t stream) {
    int idx = g_mx_tile_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= mx_tile_config_count()) {
        if (offsets) {
            // grouped: 64 x 256 tiles (MoE shape, 64 rows per expert on average:
            // 33.7 us against 37.1 for 32 x 256 and 40.6-71.8 for the others);
            // 32-row tiles when experts average at most 32 rows
            idx = M / E <= 32 ? 5 : 4;
        } else {
            const auto items = [&](int bm, int bn) { return (M + bm - 1) / bm * ((N + bn - 1) / bn); };
            idx = items(32, 256) <= 512 ? 5 : items(64, 256) <= 512 ? 4 : items(128, 512) <= 512 ? 7 : 0;
        }
    }
    // a wave's columns must be all in or all out of N
    if (N % (kMxTileCfgs[idx].bn / kMxTileCfgs[idx].wn) != 0) idx = 0;
    const MxTileCfg c = kMxTileCfgs[idx];
#define W4_MXT(BMV, BNV, WMV, WNV)                                                                     \
    if (c.bm == BMV && c.bn == BNV && c.wm == WMV && c.wn == WNV)                                      \
        return mx_tile_launch<DT, BMV, BNV, WMV, WNV>(qx, sx, offsets, wp, y, M, K, N, E, stream);
    W4_MXT(64, 256, 1, 4) W4_MXT(128, 256, 2, 4) W4_MXT(128, 128, 2, 2) W4_MXT(64, 128, 1, 2)
    W4_MXT(128, 256, 1, 4) W4_MXT(32, 256, 1, 4) W4_MXT(256, 256, 2, 4) W4_MXT(128, 512, 1, 8)
#undef W4_MXT
    return hipErrorInvalidValue;
}

hipError_t launch_mx_gemm_tile(const void *qx, const void *sx, const void *wp, void *y, int64_t M, int64_t K,
                               int64_t N, int dt, hipStream_t stream, const int32_t *offsets, int64_t E) {
    if (M == 0) return hipSuccess;
    return dt == DT_BF16 ? mx_tile_dispatch<DT_BF16>(qx, sx, offsets, wp, y, M, K, N, E, stream)
                         : mx_tile_dispatch<DT_F16>(qx, sx, offsets, wp, y, M, K, N, E, stream);
}

}  // namespace w4
