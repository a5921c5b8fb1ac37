// gemm_tile.hip — large-M W4A16 GEMM and its grouped (MoE) form.
//
// Workgroup tile BM x BN over the whole K range; WM x WN waves, each owning a
// TM x TN = (BM/WM) x (BN/WN) sub-tile computed with 32x32x16 matrix-core
// steps in fp32.
//  * Activations: the BM x 128 slice of x for one group is staged in LDS
//    (double-buffered; the next group's slice is fetched into registers while
//    the current one is multiplied).  Rows are padded to a 304-byte (bf16) /
//    272-byte (fp16) stride so the 128-bit operand reads of 8 consecutive rows
//    hit disjoint banks.
//  * Weights: every wave loads its own 32-column x 128-row fragments straight
//    from HBM/L2 into registers (two 128-bit loads per lane per 32 columns) and
//    dequantizes them into the matrix-core operand: no LDS round trip for the
//    weights (QUICK abstract: interleave offline so the dequantized weights
//    skip the shared-memory write-back).
//  * Per-group scale (design with exact integer weights inside the matrix
//    core): acc_g = sum_{k in g} x * (v - z) in fp32, y += s[g][n] * acc_g.
//    For bf16 the operand is 128 + v and the (128 + z) * sum_k x term is taken
//    out by one extra step whose A operand is the three bf16 limbs of the row's
//    group sum (computed while staging x) and whose B operand is -(128 + z).
//  * Grouped: the work items are (row tile, column block) pairs, the row tiles
//    numbered over all experts from the expert offsets (prefix sum of
//    ceil(rows_e / BM)), computed on the device so the host never reads the
//    offsets.  The hardware hands workgroup i to XCD i % 8, and each XCD has
//    its own L2; XCD x therefore takes a contiguous range of the row tiles
//    with all their column blocks, so the row tiles of one expert and the
//    expert's weights stay in one L2 (two where a range boundary splits an
//    expert).  With 32-row tiles some items are "half items" (tile_plan):
//    two wave pairs split the item's K groups over half its columns, which
//    fills the last round of resident workgroups.  With another XCD count
//    the map still covers every output once, only the locality changes.
//    Surplus workgroups exit at once.
// Matrix-core mapping (v_mfma_f32_32x32x16_*): lane l feeds row/column l % 32
// and k-block l / 32 (64 rows of the group: chunks 2*(l/32) and 2*(l/32)+1 of
// the prepacked slot layout); result register r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32.
//  * Scale groups of 32 or 64 rows (GR = 32 or 64, weights in the
//    group-aligned layout: word t of slot L holds rows 32*t + 8*(L/16) + i):
//    step s (0..7) takes word s/2 of the lane's slot 2*(l/32) + s%2, i.e. rows
//    32*(s/2) + 16*(l/32) + 8*(s%2) + i, so steps 2h and 2h+1 cover exactly the
//    32 rows of block h.  Each scale group's steps form their own chain, whose
//    fp32 sum takes that group's scale; for bf16 each chain starts from its
//    own correction step, whose A operand holds the three bf16 limbs of every
//    32/64-row block's row sum (limbs v of block h in k-slot 3h + v).
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

// XCDs of an MI355X; workgroups are dispatched to them round-robin.
constexpr int kXcds = 8;

// LDS row stride (bytes) of the staged x slice
constexpr int tile_rowb(int dt) { return (kGroup + (dt == DT_BF16 ? 16 : 0)) * 2 + 16; }

// The work of one workgroup item: a BM x BN tile (BM x BN/2 outputs with the
// SiLU epilogue) over the K groups of this wave's share.  KS = 1: the four (or
// WM x WN) waves split the columns and run every group.  KS = 2 (a "half
// item"): waves 0-1 and 2-3 are two sub-workgroups over the same BN/2 columns,
// each over one half of the groups with its own x buffers; the halves meet at
// every barrier (the shorter half runs one empty step when the group count is
// odd) and their sums are added in LDS at the end.
template <int DT, bool ZERO, int BM, int BN, int WM, int WN, bool GROUPED, bool SILU, int GR, int KS>
__device__ __forceinline__ void tile_body(const uint16_t *__restrict__ x, const int32_t *__restrict__ row_src,
                                          const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
                                          const uint8_t *__restrict__ zero, uint16_t *__restrict__ y, int64_t K,
                                          int64_t N, int gm, const float *__restrict__ cs,
                                          const float *__restrict__ cz, uint8_t *lds_all, int64_t row0,
                                          int64_t row_end, int64_t n0, int64_t e, int wm, int wn, int kh) {
    constexpr int NT = WM * WN * 64;
    constexpr int NTS = NT / KS;                                // threads staging one x slice
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int RT = TM / 32, CT = TN / 32;
    constexpr bool CORR = DT == DT_BF16;
    constexpr int ROWB = tile_rowb(DT);                         // LDS row stride (bytes)
    constexpr int XP = BM * 16 / NTS;                           // 16-byte x chunks per thread
    static_assert(KS == 1 || KS == 2, "whole items or K halves");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert((BM * 16) % NTS == 0, "x staging must divide evenly");
    static_assert(XP <= 16, "one row-sum split per lane");
    static_assert(!SILU || (GROUPED && CT == 2), "SiLU epilogue: grouped, gate and up tile per wave");
    static_assert(GR == 0 || GR == 32 || GR == 64, "standard layout, or 32/64-row scale groups");
    static_assert(GR == 0 || !SILU, "the fused-experts chain keeps 128-row groups");
    static_assert(KS == 1 || GR == 0, "K halves use the standard layout");
    constexpr int NSUB = GR ? kGroup / GR : 1;   // scale groups per 128-row tile
    constexpr int SPS = 8 / NSUB;                // 32x32x16 steps per scale group
    constexpr int CPS = GR / 8;                  // 16-byte x chunks per scale group (GR > 0)
    constexpr int TNO = SILU ? 32 : TN;          // output columns per wave

    const int tid = threadIdx.x, lane = tid & 63;
    const int stid = tid % NTS;                  // thread index within this sub-workgroup
    uint8_t *lds = lds_all + kh * 2 * BM * ROWB;
    const int G = (int)(K / kGroup);
    const int64_t NBLK = N / 16;
    const int64_t NOUT = SILU ? N / 2 : N;       // output columns (row stride of y)
    // this wave's groups: [gb, ge), nsteps steps (equal for both K halves)
    const int nsteps = KS == 1 ? G : (G + 1) / 2;
    const int gb = kh * nsteps, ge = gb + nsteps < G ? gb + nsteps : G;
    // any group index past the share re-reads its last group (or, for an empty
    // share, the last group of K): loads stay in bounds and unconditional
    auto gclamp = [&](int g) { return g < ge ? g : (ge > gb ? ge - 1 : G - 1); };
    // A wave whose columns lie past N (N % 64 == 0, so a wave's columns are all
    // in or all out) still runs the loop on the last columns, with every load
    // in bounds, and stores nothing: no branch around any load in the loop.
    const bool wave_cols = n0 + (int64_t)wn * TNO < NOUT;
    const int64_t wcol0 = wave_cols ? n0 + (int64_t)wn * TNO : NOUT - TNO;

    // one scale (and zero) row per gm consecutive 128-row groups, or NSUB per
    // 128-row group
    const int64_t GS = GR ? (int64_t)G * NSUB : G / gm;
    const uint16_t *sc = scale + e * GS * N;
    const uint8_t *zp = ZERO ? zero + e * GS * (N / 2) : nullptr;
    const uint8_t *we = wp + e * NBLK * (int64_t)G * kTileBytes;

    // ---- activation staging -------------------------------------------------
    // Rows past the tile's end read the last valid row (finite data whose
    // result rows are never stored).
    // Each lane stages the same rows in every group: their addresses are
    // formed once.  With row_src the tile's row r reads x row row_src[r] (the
    // gather of a routed token folded into the load).
    u32x4_t xr[XP];
    const uint16_t *xrow[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int id = p * NTS + stid, r = id >> 4, c16 = id & 15;
        const int64_t grow = row0 + r < row_end ? row0 + r : row_end - 1;
        const int64_t src = row_src ? (int64_t)row_src[grow] : grow;
        xrow[p] = x + src * K + c16 * 8;
    }
    auto load_x = [&](int g) {
#pragma unroll
        for (int p = 0; p < XP; ++p) xr[p] = ld128(xrow[p] + (int64_t)g * kGroup);
    };
    // Sum of a value over the 16 lanes of a row (lanes 16i .. 16i+15) with
    // row rotations: every lane ends with the row's sum.
    auto row16_sum = [](float v) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
        return v;
    };
    // x slice into LDS; for bf16 also the three bf16 limbs of each row's sum
    // (16 lanes hold a row's 16 chunks; after the row reduction every lane of
    // the row has the sum, and lane c16 = p splits and stores the sum of its
    // p-th row, so each lane splits one sum).  The 16 bytes after the limbs
    // are zero (written once before the loop).
    auto store_x = [&](int buf) {
        uint8_t *base = lds + buf * BM * ROWB;
        float ps[XP];
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int id = p * NTS + stid, r = id >> 4, c16 = id & 15;
            *reinterpret_cast<u32x4_t *>(base + r * ROWB + c16 * 16) = xr[p];
            if constexpr (CORR) {
                const bf16x2_t ones = as<bf16x2_t>(0x3F803F80u);
                float v = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v = __builtin_amdgcn_fdot2_f32_bf16(as<bf16x2_t>(xr[p][q]), ones, v, false);
                if constexpr (GR == 0) {
                    ps[p] = row16_sum(v);
                } else {
                    // sum over the CPS lanes (chunks) of one 32/64-row block
                    v += __shfl_xor(v, 1);
                    v += __shfl_xor(v, 2);
                    if constexpr (CPS == 8) v += __shfl_xor(v, 4);
                    ps[p] = v;
                }
            }
        }
        if constexpr (CORR && GR == 0) {
            const int c16 = stid & 15;
            float mine = ps[0];
#pragma unroll
            for (int p = 1; p < XP; ++p) mine = c16 == p ? ps[p] : mine;
            uint32_t hi, mid, lo;
            split3_bf16(mine, hi, mid, lo);
            if (c16 < XP) {
                const int r = (c16 * NTS + stid) >> 4;
                *reinterpret_cast<u32x4_t *>(base + r * ROWB + 256) = u32x4_t{hi | (mid << 16), lo, 0, 0};
            }
        }
        if constexpr (CORR && GR != 0) {
            // the first lane of each block stores its block's limbs: k-slots
            // 3h, 3h + 1, 3h + 2 (bytes 256 + 6h ..)
            const int c16 = stid & 15;
            if (c16 % CPS == 0) {
                const int h = c16 / CPS;
#pragma unroll
                for (int p = 0; p < XP; ++p) {
                    const int r = (p * NTS + stid) >> 4;
                    uint32_t hi, mid, lo;
                    split3_bf16(ps[p], hi, mid, lo);
                    uint16_t *lp = reinterpret_cast<uint16_t *>(base + r * ROWB + 256 + 6 * h);
                    lp[0] = (uint16_t)hi;
                    lp[1] = (uint16_t)mid;
                    lp[2] = (uint16_t)lo;
                }
            }
        }
    };
    if constexpr (CORR) {
        // k-slots past the limbs read as zero: bytes 272.. (one sum) or
        // 256 + 6 * NSUB .. 287 (per-block sums), written once
        for (int r = stid; r < 2 * BM; r += NTS) {
            if constexpr (GR == 0) {
                *reinterpret_cast<u32x4_t *>(lds + r * ROWB + 272) = u32x4_t{0, 0, 0, 0};
            } else {
                uint16_t *lp = reinterpret_cast<uint16_t *>(lds + r * ROWB + 256);
                for (int k = 3 * NSUB; k < 16; ++k) lp[k] = 0;
            }
        }
    }

    // ---- weight fragments, scales and zero points -----------------------------
    const int lj = lane & 31, kg = lane >> 5;
    // weight column of this lane in column tile ct
    auto wcol = [&](int ct) -> int64_t { return wcol0 + (SILU ? ct * NOUT : ct * 32) + lj; };
    int64_t boff[CT];          // byte offset of this lane's slot (chunk 2*kg) in group 0
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int64_t n = wcol(ct);
        const int64_t nb = n >> 4, jj = n & 15;
        boff[ct] = nb * (int64_t)G * kTileBytes + ((2 * kg) * 16 + jj) * 16;
    }
    u32x4_t braw[CT][2], bnext[CT][2];
    // scales and zero points stay in their loaded 16/8-bit types: a mask of
    // the loaded value would be a use of the load, and the compiler may place
    // it right after the prefetch (forcing a wait for every load in flight)
    uint16_t sraw[CT][NSUB], snext[CT][NSUB];
    uint8_t zraw[CT][NSUB], znext[CT][NSUB];
    auto load_b = [&](int g, u32x4_t (&dst)[CT][2], uint16_t (&sdst)[CT][NSUB], uint8_t (&zdst)[CT][NSUB]) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const uint8_t *p = we + boff[ct] + (int64_t)g * kTileBytes;
            dst[ct][0] = ld128(p);
            dst[ct][1] = ld128(p + 256);     // chunk 2*kg + 1: 16 slots further
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t n = wcol(ct);
#pragma unroll
            for (int h = 0; h < NSUB; ++h) {
                const int64_t gs = GR ? (int64_t)g * NSUB + h : g / gm;
                sdst[ct][h] = sc[gs * N + n];
                zdst[ct][h] = ZERO ? zp[(gs * N + n) >> 1] : (uint8_t)0;
            }
        }
    };

    f32x16_t yacc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[rt][ct][r] = 0.f;

    load_x(gclamp(gb));
    load_b(gclamp(gb), braw, sraw, zraw);
    store_x(0);
    __syncthreads();

    // Every step issues the loads of the next group first (the last step
    // re-reads group G - 1: no branch, so the counters of outstanding loads
    // stay exact and each wait covers only what is used), multiplies the
    // current group from registers and LDS, then stages the next x slice.
    // Two register sets for the weights, scales and zero points alternate
    // between steps, so a prefetch is waited for only in the step that uses
    // it (a register copy would wait for it at once).
    const int arow = wm * TM + lj;             // LDS row of this lane's A operand (row tile 0)
    constexpr int kStageStep = 4;              // k-step after which the next x slice is staged
    auto step = [&](int gi, const u32x4_t (&bw)[CT][2], const uint16_t (&sw)[CT][NSUB],
                    const uint8_t (&zw)[CT][NSUB], u32x4_t (&bn)[CT][2], uint16_t (&sn)[CT][NSUB],
                    uint8_t (&zn)[CT][NSUB]) {
        const int buf = gi & 1;
        const bool valid = gb + gi < ge;           // uniform: the shorter K half's last step is empty
        const int gn = gclamp(gb + gi + 1);
        load_x(gn);
        load_b(gn, bn, sn, zn);
        const uint8_t *abase = lds + buf * BM * ROWB + arow * ROWB + (GR ? kg * 32 : kg * 128);
        // A operand of the correction steps: the bf16 limbs of the rows' sums
        u32x4_t alimb[RT];
        if constexpr (CORR) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                alimb[rt] = *reinterpret_cast<const u32x4_t *>(lds + buf * BM * ROWB + (arow + rt * 32) * ROWB + 256 +
                                                               kg * 16);
        }
#pragma unroll
        for (int h = 0; h < NSUB; ++h) {
            float s[CT];
            uint32_t nb2[CT];
            u32x4_t bcorr[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int64_t n = wcol(ct);
                s[ct] = h2f<DT>(sw[ct][h]);
                uint32_t z = 8;
                if constexpr (ZERO) z = __builtin_amdgcn_ubfe((uint32_t)zw[ct][h], (uint32_t)(n & 1) * 4u, 4);
                if constexpr (CORR) {
                    const uint32_t c = bf16_negbias(z);
                    if constexpr (GR == 0) {
                        bcorr[ct] = kg == 0 ? u32x4_t{c | (c << 16), c, 0, 0} : u32x4_t{0, 0, 0, 0};
                    } else {
                        // c in k-slots 3h .. 3h + 2 only; this lane holds slots
                        // 8*kg .. 8*kg + 7, two per word
                        const uint32_t cc = c | (c << 16);
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            constexpr uint32_t lo16 = 0x0000FFFFu, hi16 = 0xFFFF0000u;
                            auto msk = [&](int slot) -> uint32_t {
                                return (slot >= 3 * h && slot < 3 * h + 3) ? ((slot & 1) ? hi16 : lo16) : 0u;
                            };
                            const uint32_t m0 = msk(2 * w) | msk(2 * w + 1);
                            const uint32_t m1 = msk(8 + 2 * w) | msk(8 + 2 * w + 1);
                            bcorr[ct][w] = cc & (kg == 0 ? m0 : m1);
                        }
                    }
                    nb2[ct] = 0;
                } else {
                    nb2[ct] = f16_negbias2(z);
                }
            }
            // accumulator inputs of the first step: the bias correction (bf16; one
            // per row tile when every column has z = 8, else one per column tile)
            // or zero.  Passing it as the matrix-core C input avoids copying one
            // correction into several accumulators.
            f32x16_t cin[RT][ZERO ? CT : 1];
            if constexpr (CORR) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ci = 0; ci < (ZERO ? CT : 1); ++ci)
                        cin[rt][ci] = mfma32x32x16<DT>(alimb[rt], bcorr[ci], f32x16_t{});
            }
            f32x16_t acc[RT][CT];
#pragma unroll
            for (int t = h * SPS; t < (h + 1) * SPS; ++t) {
                u32x4_t a[RT], bq[CT];
                // k offset of this step's operands: 8t (standard layout) or
                // 32*(t/2) + 16*kg + 8*(t%2) (group-aligned; kg part in abase)
                const int aoff = GR ? (t >> 1) * 64 + (t & 1) * 16 : t * 16;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    a[rt] = *reinterpret_cast<const u32x4_t *>(abase + rt * 32 * ROWB + aoff);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    bq[ct] = GR ? dequant_word<DT>(bw[ct][t & 1][t >> 1], nb2[ct])
                                : dequant_word<DT>(bw[ct][t >> 2][t & 3], nb2[ct]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        if (t == h * SPS) {
                            if constexpr (CORR) acc[rt][ct] = mfma32x32x16<DT>(a[rt], bq[ct], cin[rt][ZERO ? ct : 0]);
                            else acc[rt][ct] = mfma32x32x16<DT>(a[rt], bq[ct], f32x16_t{});
                        } else {
                            acc[rt][ct] = mfma32x32x16<DT>(a[rt], bq[ct], acc[rt][ct]);
                        }
                    }
                // stage the next group's x slice halfway through the products: its
                // vector work (row sums, limb split) then overlaps matrix-core
                // steps.  The buffer written was last read in the previous step,
                // before that step's barrier.
                if (t == kStageStep) store_x(buf ^ 1);
            }
            if (valid) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int r = 0; r < 16; ++r) yacc[rt][ct][r] += s[ct] * acc[rt][ct][r];
            }
        }
        __syncthreads();
    };
    for (int gi = 0; gi < nsteps; gi += 2) {
        step(gi, braw, sraw, zraw, bnext, snext, znext);
        if (gi + 1 < nsteps) step(gi + 1, bnext, snext, znext, braw, sraw, zraw);
    }

    if constexpr (KS == 2) {
        // sum of the two K halves, in LDS (the x buffers are free: every wave
        // has passed the barrier after its last read of them): the second
        // half's waves store their sums, the first half's waves add them in
        // a fixed order and run the epilogue
        float *red = reinterpret_cast<float *>(lds_all);
        auto slot = [&](int rt, int ct, int q) { return red + ((((wn * RT + rt) * CT + ct) * 4 + q) * 64 + lane) * 4; };
        if (kh == 1) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<f32x4_t *>(slot(rt, ct, q)) =
                            f32x4_t{yacc[rt][ct][4 * q], yacc[rt][ct][4 * q + 1], yacc[rt][ct][4 * q + 2],
                                    yacc[rt][ct][4 * q + 3]};
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4_t v = *reinterpret_cast<const f32x4_t *>(slot(rt, ct, q));
#pragma unroll
                    for (int i = 0; i < 4; ++i) yacc[rt][ct][4 * q + i] += v[i];
                }
    }

    if (!wave_cols) return;
    if constexpr (SILU) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int64_t col = wcol0 + lj;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = row0 + wm * TM + rt * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
                if (row < row_end) {
                    const float gf = h2f<DT>(f2h<DT>(yacc[rt][0][r]));
                    const float uf = h2f<DT>(f2h<DT>(yacc[rt][1][r]));
                    const float sg = gf / (1.0f + expf(-gf));
                    y[row * NOUT + col] = f2h<DT>(sg * uf);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t col = wcol0 + ct * 32 + lj;
            const float t = cs ? cs[col] : 1.f;           // secondary (per-column) scale
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = row0 + wm * TM + rt * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
                if (row < row_end) {
                    float v = yacc[rt][ct][r];
                    if (cz) v -= cz[row * N + col];       // floating-point zero points
                    y[row * N + col] = f2h<DT>(cs ? v * t : v);
                }
            }
        }
}

// Half items (grouped 32 x 256 tiles, four waves of 32 x 64): the planner
// below may split an item's K range between two wave pairs, each over half
// the item's columns, so that a half item takes about half the time of a
// whole one.  The hardware keeps a fixed number of workgroups resident (three
// per compute unit for these tiles); when the whole items overrun a round by
// a few, the rest of the machine would otherwise idle through a second round.
template <int BM, int WM, int WN, bool GROUPED, int GR>
constexpr bool tile_half_ok() {
    return GROUPED && GR == 0 && BM == 32 && WM == 1 && WN == 4;
}

// Finishing time, in half-item durations, of F whole and H half items
// dispatched in that order onto S slots (each whole item two units).
__device__ __forceinline__ int64_t tile_makespan(int64_t F, int64_t H, int64_t S) {
    const int64_t q = F / S, r = F % S;
    if (r == 0) return 2 * q + (H + S - 1) / S;
    const int64_t rem = H - 2 * (S - r);       // halves the partly used round cannot take
    return 2 * q + 2 + (rem > 0 ? (rem + S - 1) / S : 0);
}

struct TileItem {
    int64_t tile, ncol;   // global row tile, first output column
    int half, valid;
};

// Item k (dispatch order) of XCD xcd.  XCD x owns the contiguous row tiles
// [T*x/8, T*(x+1)/8) with all their column blocks, so an expert's row tiles
// share one L2 (two where the boundary splits it).  Its list holds the whole
// items first, in (row tile, column block) order, then the half items: the
// two halves of each of the last c whole items (c chosen to shorten the
// finishing time on S resident slots per XCD, else 0), then the last column
// block of every row tile when it spans at most half a block.  Every output
// column of every row tile is covered exactly once.
__device__ __forceinline__ TileItem tile_plan(int64_t T, int64_t xcd, int64_t k, int64_t ncb, int64_t bno,
                                              int64_t nout, int64_t S, bool halfok) {
    TileItem it{0, 0, 0, 0};
    const int64_t t0 = T * xcd / kXcds, t1 = T * (xcd + 1) / kXcds, nt = t1 - t0;
    const int64_t lastw = nout - (ncb - 1) * bno;
    halfok = halfok && S > 0;
    const int64_t nh = (halfok && 2 * lastw <= bno) ? 1 : 0, nfb = ncb - nh;
    const int64_t F0 = nt * nfb, H0 = nt * nh;
    int64_t c = 0;
    if (halfok) {
        const int64_t r = F0 % S;
        if (r > 0 && tile_makespan(F0 - r, H0 + 2 * r, S) < tile_makespan(F0, H0, S)) c = r;
    }
    const int64_t F = F0 - c, H = H0 + 2 * c;
    if (k < F) {
        it.tile = t0 + k / nfb;
        it.ncol = (k % nfb) * bno;
        it.valid = 1;
    } else if (k < F + H) {
        const int64_t j = k - F;
        if (j < 2 * c) {
            const int64_t fi = F + j / 2;
            it.tile = t0 + fi / nfb;
            it.ncol = (fi % nfb) * bno + (j & 1) * (bno / 2);
        } else {
            it.tile = t0 + (j - 2 * c);
            it.ncol = (ncb - 1) * bno;
        }
        it.half = 1;
        it.valid = 1;
    }
    return it;
}

// At least two waves per SIMD: two resident workgroups of four waves (or one
// of eight) per compute unit, each wave within 256 registers.
//
// SILU (grouped, two 32-column tiles per wave): the weights hold 2 * NOUT
// columns, gate then up (the fused-experts gate/up projection); a wave's two
// tiles are gate columns c and up columns NOUT + c of the same 32 output
// columns, and the epilogue stores a = silu(gate) * up with each input first
// rounded to the activation dtype (as if the projection were stored and read
// back), so the result equals that of the separate SiLU-and-multiply kernel.
// slots: resident workgroups per XCD, for the item plan (any value >= 1 gives
// results within the same bound; 0 plans no half items).
template <int DT, bool ZERO, int BM, int BN, int WM, int WN, bool GROUPED, bool SILU = false, int GR = 0>
__global__ void __launch_bounds__(WM * WN * 64, 2)
gemm_tile_kernel(const uint16_t *__restrict__ x, const int32_t *__restrict__ offsets,
                 const int32_t *__restrict__ row_src, const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
                 const uint8_t *__restrict__ zero, uint16_t *__restrict__ y,
                 int64_t M, int64_t K, int64_t N, int E, int gm, const float *__restrict__ cs,
                 const float *__restrict__ cz, int slots) {
    constexpr int NT = WM * WN * 64;
    constexpr int ROWB = tile_rowb(DT);
    constexpr bool HALF = tile_half_ok<BM, WM, WN, GROUPED, GR>();
    constexpr int BNO = SILU ? BN / 2 : BN;   // output columns per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t lds[(HALF ? 2 : 1) * 2 * BM * ROWB];

    // the wave index is uniform (readfirstlane: values derived from it stay
    // in scalar registers)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t NOUT = SILU ? N / 2 : N;

    int64_t row0, row_end, n0;
    int64_t e = 0;
    bool half = false;
    if constexpr (GROUPED) {
        __shared__ int s_info[6];              // expert, row tile within it, first column, half, its offsets
        __shared__ int s_total;
        __shared__ int scan[NT];
        // row tiles of expert ee (0 past E); o0, o1 get its offsets
        auto tiles_of = [&](int ee, int &o0, int &o1) {
            o0 = ee < E ? offsets[ee] : 0;
            o1 = ee < E ? offsets[ee + 1] : 0;
            const int cnt = o1 - o0;
            return cnt > 0 ? (cnt + BM - 1) / BM : 0;
        };
        const int64_t ncb = (NOUT + BNO - 1) / BNO;
        const int64_t bid = blockIdx.x, xcd = bid % kXcds, k = bid / kXcds;
        if (E <= 64) {
            // one wave: inclusive scan of the experts' row tiles over its
            // lanes, the plan, then the expert holding this item's row tile
            if (wave == 0) {
                int o0, o1;
                const int tl = tiles_of(lane, o0, o1);
                const int incl = wave_incl_scan(tl);
                const int64_t total = __builtin_amdgcn_readlane(incl, 63);
                const TileItem it = tile_plan(total, xcd, k, ncb, BNO, NOUT, slots, HALF);
                if (lane == 0) {
                    s_info[0] = -1;
                    s_info[2] = (int)it.ncol;
                    s_info[3] = it.half;
                }
                if (it.valid && lane < E && it.tile >= incl - tl && it.tile < incl) {
                    s_info[0] = lane;
                    s_info[1] = (int)(it.tile - (incl - tl));
                    s_info[4] = o0;
                    s_info[5] = o1;
                }
            }
            __syncthreads();
        } else {
        // total row tiles over all experts
        if (tid == 0) {
            s_info[0] = -1;
            s_total = 0;
        }
        __syncthreads();
        int part = 0;
        for (int ee = tid; ee < E; ee += NT) {
            int o0, o1;
            part += tiles_of(ee, o0, o1);
        }
        part = __builtin_amdgcn_readlane(wave_incl_scan(part), 63);
        if (lane == 0) atomicAdd(&s_total, part);
        __syncthreads();
        const TileItem it = tile_plan(s_total, xcd, k, ncb, BNO, NOUT, slots, HALF);
        if (!it.valid) return;   // uniform: surplus workgroup
        if (tid == 0) {
            s_info[2] = (int)it.ncol;
            s_info[3] = it.half;
        }
        const int tile = (int)it.tile;
        // expert and row tile within it (block-wide inclusive scan per chunk)
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
                s_info[4] = o0;
                s_info[5] = o1;
            }
            carry += scan[NT - 1];
            __syncthreads();
        }
        }
        const int es = __builtin_amdgcn_readfirstlane(s_info[0]);
        if (es < 0) return;      // uniform: surplus workgroup
        e = es;
        const int64_t tin = __builtin_amdgcn_readfirstlane(s_info[1]);
        n0 = __builtin_amdgcn_readfirstlane(s_info[2]);
        half = __builtin_amdgcn_readfirstlane(s_info[3]) != 0;
        // the expert's offsets as its scan lane read them (no second load)
        const int64_t oe = __builtin_amdgcn_readfirstlane(s_info[4]);
        const int64_t oe1 = __builtin_amdgcn_readfirstlane(s_info[5]);
        row0 = oe + tin * BM;
        row_end = oe1 < M ? oe1 : M;   // offsets[E] == R by contract
    } else {
        row0 = (int64_t)blockIdx.x * BM;
        row_end = M;
        n0 = (int64_t)blockIdx.y * BN;
    }
    if constexpr (HALF) {
        if (half) {
            tile_body<DT, ZERO, BM, BN, WM, WN, GROUPED, SILU, GR, 2>(x, row_src, wp, scale, zero, y, K, N, gm, cs, cz,
                                                                      lds, row0, row_end, n0, e, 0, wave & 1,
                                                                      wave >> 1);
            return;
        }
    }
    tile_body<DT, ZERO, BM, BN, WM, WN, GROUPED, SILU, GR, 1>(x, row_src, wp, scale, zero, y, K, N, gm, cs, cz, lds,
                                                              row0, row_end, n0, e, wave / WN, wave % WN, 0);
}

// Workgroup tile configurations (BM x BN rows x columns, WM x WN waves).
// Index 0 is the dense default for large M: 64 x 64 wave tiles in workgroups
// of four waves, two resident per compute unit, so that one workgroup's
// matrix-core steps overlap the other's vector work across their separate
// per-group barriers (measured ~5% faster on 4096^3 than one eight-wave
// 128 x 256 workgroup with the same wave tile).  Smaller M takes indices 4
// and 2 by workgroup count (see the dispatcher).  The grouped default follows
// the average row count per expert (small row tiles waste less of the matrix
// core on experts with few rows).  The others are kept for tuning through the
// test hook.
struct TileCfg { int bm, bn, wm, wn; };
static constexpr TileCfg kTileCfgs[] = {{64, 256, 1, 4}, {64, 256, 2, 4}, {32, 256, 1, 4},
                                        {64, 128, 2, 2}, {32, 128, 1, 4}, {128, 128, 2, 2},
                                        {128, 256, 2, 4}, {64, 128, 1, 2}};
static std::atomic<int> g_tile_cfg{-1};      // -1: automatic
static std::atomic<int> g_tile_halves{1};    // half items allowed (test hook)
int set_tile_halves(int enable) { return g_tile_halves.exchange(enable ? 1 : 0, std::memory_order_relaxed); }

int tile_config_count() { return (int)(sizeof(kTileCfgs) / sizeof(kTileCfgs[0])); }
void set_tile_config(int idx) { g_tile_cfg.store(idx, std::memory_order_relaxed); }

template <int DT, bool ZERO, bool GROUPED, int BM, int BN, int WM, int WN, bool SILU = false, int GR = 0>
static hipError_t tile_launch(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                              const void *scale, const void *zero, void *y, int64_t M, int64_t K, int64_t N,
                              int64_t E, int gm, const float *cs, const float *cz, hipStream_t stream) {
    constexpr bool HALF = tile_half_ok<BM, WM, WN, GROUPED, GR>();
    auto kern = gemm_tile_kernel<DT, ZERO, BM, BN, WM, WN, GROUPED, SILU, GR>;
    const int64_t ncb = SILU ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
    const int64_t mtiles = GROUPED ? (M + BM - 1) / BM + E : (M + BM - 1) / BM;
    int sx = 1;
    if (GROUPED && HALF && !g_tile_halves.load(std::memory_order_relaxed)) {
        sx = 0;                          // no half items
    } else if constexpr (GROUPED) {
        // resident workgroups per XCD, for the item plan (queried once; a
        // failed query only makes the plan less balanced)
        static std::atomic<int> cached{0};
        sx = cached.load(std::memory_order_relaxed);
        if (sx <= 0) {
            // (an error of these queries is cleared so that it is not reported
            // by the launch below; nothing else touches the error state)
            int dev = 0, cus = 0, blocks = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
                (void)hipGetLastError();
                cus = 256;
            }
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void *>(kern),
                                                             WM * WN * 64, 0) != hipSuccess) {
                (void)hipGetLastError();
                blocks = 1;
            }
            if (cus < 1) cus = 256;
            if (blocks < 1) blocks = 1;
            sx = cus * blocks / kXcds > 0 ? cus * blocks / kXcds : 1;
            cached.store(sx, std::memory_order_relaxed);
        }
    }
    // grouped: every expert may end in a partial row tile, hence + E; each XCD
    // takes at most ceil(mtiles / 8) row tiles with all their column blocks,
    // plus fewer than sx extra half items; the grid holds that many slots per
    // XCD (surplus workgroups exit at once)
    const int64_t per_xcd = (mtiles + kXcds - 1) / kXcds * ncb + (HALF && sx > 0 ? sx : 0);
    const int64_t slots = per_xcd * kXcds;
    if (GROUPED && slots > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid = GROUPED ? dim3((unsigned)slots) : dim3((unsigned)mtiles, (unsigned)ncb);
    hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), 0, stream, (const uint16_t *)x, offsets, row_src,
                       (const uint8_t *)wp, (const uint16_t *)scale, (const uint8_t *)zero, (uint16_t *)y, M, K, N,
                       (int)E, gm, cs, cz, sx);
    return hipGetLastError();
}

template <int DT, bool ZERO, bool GROUPED>
static hipError_t tile_dispatch(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                                const void *scale, const void *zero, void *y, int64_t M, int64_t K, int64_t N,
                                int64_t E, int gm, const float *cs, const float *cz, hipStream_t stream) {
    int idx = g_tile_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= tile_config_count()) {
        idx = 0;
        if (GROUPED) {
            // few rows per expert: 32-row tiles (little padding); 32 x 256
            // measured best on the MoE shapes (fused-experts chain 173-177 us
            // against 190-194 us with 32 x 128; grouped call about even)
            const int64_t avg = M / E;          // mean rows per expert
            idx = avg <= 96 ? 2 : 0;
        } else {
            // M ranges by workgroup count (measured over M = 17..4096 at
            // K = 4096, N = 4096 and 14336): while 32 x 128 tiles give at most
            // 672 workgroups they win (up to 2x against 64 x 256, which would
            // leave most compute units idle); then 32 x 256 while 64 x 256
            // would give fewer than 448; 64 x 256 beyond
            const int64_t items4 = (M + 31) / 32 * ((N + 127) / 128);
            const int64_t items0 = (M + 63) / 64 * ((N + 255) / 256);
            idx = items4 <= 672 ? 4 : (items0 < 448 ? 2 : 0);
        }
    }
    const TileCfg c = kTileCfgs[idx];
#define W4_TILE(BMV, BNV, WMV, WNV)                                                                    \
    if (c.bm == BMV && c.bn == BNV && c.wm == WMV && c.wn == WNV)                                      \
        return tile_launch<DT, ZERO, GROUPED, BMV, BNV, WMV, WNV>(x, offsets, row_src, wp, scale, zero, y, M, K,   \
                                                                  N, E, gm, cs, cz, stream);
    W4_TILE(128, 256, 2, 4) W4_TILE(64, 256, 2, 4) W4_TILE(32, 256, 1, 4) W4_TILE(64, 128, 2, 2)
    W4_TILE(32, 128, 1, 4) W4_TILE(128, 128, 2, 2) W4_TILE(64, 256, 1, 4) W4_TILE(64, 128, 1, 2)
#undef W4_TILE
    return hipErrorInvalidValue;
}

template <bool GROUPED>
static hipError_t tile_dispatch_dt(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                                   const void *scale, const void *zero, void *y, int64_t M, int64_t K, int64_t N,
                                   int64_t E, int gm, int dt, const float *cs, const float *cz,
                                   hipStream_t stream) {
    if (dt == DT_BF16)
        return zero ? tile_dispatch<DT_BF16, true, GROUPED>(x, offsets, row_src, wp, scale, zero, y, M, K, N, E, gm, cs, cz, stream)
                    : tile_dispatch<DT_BF16, false, GROUPED>(x, offsets, row_src, wp, scale, zero, y, M, K, N, E, gm, cs, cz, stream);
    return zero ? tile_dispatch<DT_F16, true, GROUPED>(x, offsets, row_src, wp, scale, zero, y, M, K, N, E, gm, cs, cz, stream)
                : tile_dispatch<DT_F16, false, GROUPED>(x, offsets, row_src, wp, scale, zero, y, M, K, N, E, gm, cs, cz, stream);
}

// Grouped gate/up projection with the SiLU-and-multiply epilogue (N = 2 * I
// weight columns in, a [M][I] out) for the grouped tile shapes whose waves
// hold a gate and an up tile; hipErrorNotSupported for any other shape (the
// caller then runs the projection and the separate kernel).
template <int DT, bool ZERO>
static hipError_t tile_silu_dispatch(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                                     const void *scale, const void *zero, void *a, int64_t M, int64_t K, int64_t N,
                                     int64_t E, hipStream_t stream) {
    int idx = g_tile_cfg.load(std::memory_order_relaxed);
    if (idx < 0 || idx >= tile_config_count()) idx = M / E <= 96 ? 2 : 0;     // the grouped defaults
    const TileCfg c = kTileCfgs[idx];
    if (c.bm == 32 && c.bn == 256 && c.wm == 1 && c.wn == 4)
        return tile_launch<DT, ZERO, true, 32, 256, 1, 4, true>(x, offsets, row_src, wp, scale, zero, a, M, K, N, E,
                                                                1, nullptr, nullptr, stream);
    if (c.bm == 64 && c.bn == 256 && c.wm == 1 && c.wn == 4)
        return tile_launch<DT, ZERO, true, 64, 256, 1, 4, true>(x, offsets, row_src, wp, scale, zero, a, M, K, N, E,
                                                                1, nullptr, nullptr, stream);
    return hipErrorNotSupported;
}

hipError_t launch_gemm_tile_silu(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                                 const void *scale, const void *zero, void *a, int64_t M, int64_t K, int64_t N,
                                 int64_t E, int dt, hipStream_t stream) {
    if (dt == DT_BF16)
        return zero ? tile_silu_dispatch<DT_BF16, true>(x, offsets, row_src, wp, scale, zero, a, M, K, N, E, stream)
                    : tile_silu_dispatch<DT_BF16, false>(x, offsets, row_src, wp, scale, zero, a, M, K, N, E, stream);
    return zero ? tile_silu_dispatch<DT_F16, true>(x, offsets, row_src, wp, scale, zero, a, M, K, N, E, stream)
                : tile_silu_dispatch<DT_F16, false>(x, offsets, row_src, wp, scale, zero, a, M, K, N, E, stream);
}

// Scale groups of 32 or 64 rows (group-aligned weights): 32-row wave tiles
// (the per-scale-group chains and scales of 64-row wave tiles do not fit in
// 256 registers), 32 x 128 while that gives at most 672 workgroups (or, for
// grouped calls, experts average <= 96 rows), else 32 x 256; the tuning hook
// does not apply.
template <int DT, bool ZERO, bool GROUPED, int GR>
static hipError_t tile_gs_dispatch(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                                   const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E,
                                   const float *cs, const float *cz, hipStream_t stream) {
    const bool narrow = GROUPED ? M / E <= 96 : (M + 31) / 32 * ((N + 127) / 128) <= 672;
    if (narrow)
        return tile_launch<DT, ZERO, GROUPED, 32, 128, 1, 4, false, GR>(x, offsets, nullptr, wp, scale, zero, y, M, K,
                                                                        N, E, 1, cs, cz, stream);
    return tile_launch<DT, ZERO, GROUPED, 32, 256, 1, 4, false, GR>(x, offsets, nullptr, wp, scale, zero, y, M, K, N,
                                                                    E, 1, cs, cz, stream);
}

template <bool GROUPED, int GR>
static hipError_t tile_gs_dispatch_dt(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                                      const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E, int dt,
                                      const float *cs, const float *cz, hipStream_t stream) {
    if (dt == DT_BF16)
        return zero ? tile_gs_dispatch<DT_BF16, true, GROUPED, GR>(x, offsets, wp, scale, zero, y, M, K, N, E, cs, cz, stream)
                    : tile_gs_dispatch<DT_BF16, false, GROUPED, GR>(x, offsets, wp, scale, zero, y, M, K, N, E, cs, cz, stream);
    return zero ? tile_gs_dispatch<DT_F16, true, GROUPED, GR>(x, offsets, wp, scale, zero, y, M, K, N, E, cs, cz, stream)
                : tile_gs_dispatch<DT_F16, false, GROUPED, GR>(x, offsets, wp, scale, zero, y, M, K, N, E, cs, cz, stream);
}

hipError_t launch_gemm_tile_gs(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                               const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E, int dt,
                               int group_size, hipStream_t stream, const float *cs, const float *cz) {
    if (offsets) {
        if (group_size == 32) return tile_gs_dispatch_dt<true, 32>(x, offsets, wp, scale, zero, y, M, K, N, E, dt, cs, cz, stream);
        if (group_size == 64) return tile_gs_dispatch_dt<true, 64>(x, offsets, wp, scale, zero, y, M, K, N, E, dt, cs, cz, stream);
    } else {
        if (group_size == 32) return tile_gs_dispatch_dt<false, 32>(x, nullptr, wp, scale, zero, y, M, K, N, 1, dt, cs, cz, stream);
        if (group_size == 64) return tile_gs_dispatch_dt<false, 64>(x, nullptr, wp, scale, zero, y, M, K, N, 1, dt, cs, cz, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_tile(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                            const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E,
                            int dt, hipStream_t stream, const int32_t *row_src, int gm, const float *cs,
                            const float *cz) {
    if (offsets) return tile_dispatch_dt<true>(x, offsets, row_src, wp, scale, zero, y, M, K, N, E, gm, dt, cs, cz, stream);
    return tile_dispatch_dt<false>(x, nullptr, row_src, wp, scale, zero, y, M, K, N, 1, gm, dt, cs, cz, stream);
}

}  // namespace w4
