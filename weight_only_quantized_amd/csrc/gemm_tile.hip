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
//    its own L2; XCD x therefore takes an equal, contiguous range of the items
//    in (row tile, column block) order, so the row tiles of one expert and the
//    expert's weights stay in one L2 (two where a range boundary splits an
//    expert).  With another XCD count the map is still a bijection, only the
//    locality changes.  Surplus workgroups exit at once.
// Matrix-core mapping (v_mfma_f32_32x32x16_*): lane l feeds row/column l % 32
// and k-block l / 32 (64 rows of the group: chunks 2*(l/32) and 2*(l/32)+1 of
// the prepacked slot layout); result register r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

// XCDs of an MI355X; workgroups are dispatched to them round-robin.
constexpr int kXcds = 8;

// At least two waves per SIMD: two resident workgroups of four waves (or one
// of eight) per compute unit, each wave within 256 registers.
//
// SILU (grouped, two 32-column tiles per wave): the weights hold 2 * NOUT
// columns, gate then up (the fused-experts gate/up projection); a wave's two
// tiles are gate columns c and up columns NOUT + c of the same 32 output
// columns, and the epilogue stores a = silu(gate) * up with each input first
// rounded to the activation dtype (as if the projection were stored and read
// back), so the result equals that of the separate SiLU-and-multiply kernel.
template <int DT, bool ZERO, int BM, int BN, int WM, int WN, bool GROUPED, bool SILU = false>
__global__ void __launch_bounds__(WM * WN * 64, 2)
gemm_tile_kernel(const uint16_t *__restrict__ x, const int32_t *__restrict__ offsets,
                 const int32_t *__restrict__ row_src, const uint8_t *__restrict__ wp, const uint16_t *__restrict__ scale,
                 const uint8_t *__restrict__ zero, uint16_t *__restrict__ y,
                 int64_t M, int64_t K, int64_t N, int E, int gm, const float *__restrict__ cs,
                 const float *__restrict__ cz) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int RT = TM / 32, CT = TN / 32;
    constexpr bool CORR = DT == DT_BF16;
    constexpr int ROWB = (kGroup + (CORR ? 16 : 0)) * 2 + 16;   // LDS row stride (bytes)
    constexpr int XP = BM * 16 / NT;                            // 16-byte x chunks per thread
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert((BM * 16) % NT == 0, "x staging must divide evenly");
    static_assert(XP <= 16, "one row-sum split per lane");
    static_assert(!SILU || (GROUPED && CT == 2), "SiLU epilogue: grouped, gate and up tile per wave");
    constexpr int BNO = SILU ? BN / 2 : BN;   // output columns per workgroup
    constexpr int TNO = SILU ? 32 : TN;       // output columns per wave

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BM * ROWB];

    // the wave index is uniform (readfirstlane: values derived from it stay
    // in scalar registers)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int G = (int)(K / kGroup);
    const int64_t NBLK = N / 16;
    const int64_t NOUT = SILU ? N / 2 : N;    // output columns (row stride of y)

    int64_t row0, row_end, n0;
    int64_t e = 0;
    if constexpr (GROUPED) {
        __shared__ int s_info[3];
        __shared__ int scan[NT];
        auto tiles_of = [&](int ee) {
            const int cnt = ee < E ? offsets[ee + 1] - offsets[ee] : 0;
            return cnt > 0 ? (cnt + BM - 1) / BM : 0;
        };
        // this workgroup's item: slot bid / 8 of XCD bid % 8's contiguous range
        // of (row tile, column block) items
        const int64_t ncb = (NOUT + BNO - 1) / BNO;
        const int64_t bid = blockIdx.x, xcd = bid % kXcds;
        int64_t item, last;
        if (E <= 64) {
            // one wave: inclusive scan of the experts' row tiles over its
            // lanes, then the expert holding this item's row tile
            if (wave == 0) {
                const int tl = tiles_of(lane);
                int incl = tl;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int v = __shfl_up(incl, off);
                    if (lane >= off) incl += v;
                }
                const int64_t total = __shfl(incl, 63);
                const int64_t items = total * ncb;
                const int64_t it = items * xcd / kXcds + bid / kXcds;
                const int tile = (int)(it / ncb);
                if (lane == 0) {
                    s_info[0] = -1;
                    s_info[2] = (int)total;
                }
                if (it < items * (xcd + 1) / kXcds && lane < E && tile >= incl - tl && tile < incl) {
                    s_info[0] = lane;
                    s_info[1] = tile - (incl - tl);
                }
            }
            __syncthreads();
            const int64_t items = (int64_t)s_info[2] * ncb;
            item = items * xcd / kXcds + bid / kXcds;
            last = items * (xcd + 1) / kXcds;
            if (item >= last) return;   // uniform: surplus workgroup
        } else {
        // total row tiles over all experts
        if (tid == 0) {
            s_info[0] = -1;
            s_info[2] = 0;
        }
        __syncthreads();
        int part = 0;
        for (int ee = tid; ee < E; ee += NT) part += tiles_of(ee);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        if (lane == 0) atomicAdd(&s_info[2], part);
        __syncthreads();
        const int64_t items = (int64_t)s_info[2] * ncb;
        item = items * xcd / kXcds + bid / kXcds;
        last = items * (xcd + 1) / kXcds;
        if (item >= last) return;   // uniform: surplus workgroup
        const int tile = (int)(item / ncb);
        // expert and row tile within it (block-wide inclusive scan per chunk)
        int carry = 0;
        for (int base = 0; base < E; base += NT) {
            const int ee = base + tid;
            const int tl = tiles_of(ee);
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
            }
            carry += scan[NT - 1];
            __syncthreads();
        }
        }
        n0 = (item % ncb) * BNO;
        e = s_info[0];   // always found: tile < total row tiles
        row0 = offsets[e] + (int64_t)s_info[1] * BM;
        row_end = offsets[e + 1] < M ? offsets[e + 1] : M;   // offsets[E] == R by contract
    } else {
        row0 = (int64_t)blockIdx.x * BM;
        row_end = M;
        n0 = (int64_t)blockIdx.y * BN;
    }
    // A wave whose columns lie past N (N % 64 == 0, so a wave's columns are all
    // in or all out) still runs the loop on the last columns, with every load
    // in bounds, and stores nothing: no branch around any load in the loop.
    const bool wave_cols = n0 + (int64_t)wn * TNO < NOUT;
    const int64_t wcol0 = wave_cols ? n0 + (int64_t)wn * TNO : NOUT - TNO;

    // one scale (and zero) row per gm consecutive 128-row groups
    const int64_t GS = G / gm;
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
        const int id = p * NT + tid, r = id >> 4, c16 = id & 15;
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
            const int id = p * NT + tid, r = id >> 4, c16 = id & 15;
            *reinterpret_cast<u32x4_t *>(base + r * ROWB + c16 * 16) = xr[p];
            if constexpr (CORR) {
                const bf16x2_t ones = as<bf16x2_t>(0x3F803F80u);
                float v = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v = __builtin_amdgcn_fdot2_f32_bf16(as<bf16x2_t>(xr[p][q]), ones, v, false);
                ps[p] = row16_sum(v);
            }
        }
        if constexpr (CORR) {
            const int c16 = tid & 15;
            float mine = ps[0];
#pragma unroll
            for (int p = 1; p < XP; ++p) mine = c16 == p ? ps[p] : mine;
            uint32_t hi, mid, lo;
            split3_bf16(mine, hi, mid, lo);
            if (c16 < XP) {
                const int r = (c16 * NT + tid) >> 4;
                *reinterpret_cast<u32x4_t *>(base + r * ROWB + 256) = u32x4_t{hi | (mid << 16), lo, 0, 0};
            }
        }
    };
    if constexpr (CORR) {
        for (int r = tid; r < 2 * BM; r += NT)
            *reinterpret_cast<u32x4_t *>(lds + r * ROWB + 272) = u32x4_t{0, 0, 0, 0};
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
    uint16_t sraw[CT], snext[CT];
    uint8_t zraw[CT], znext[CT];
    auto load_b = [&](int g, u32x4_t (&dst)[CT][2], uint16_t (&sdst)[CT], uint8_t (&zdst)[CT]) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const uint8_t *p = we + boff[ct] + (int64_t)g * kTileBytes;
            dst[ct][0] = ld128(p);
            dst[ct][1] = ld128(p + 256);     // chunk 2*kg + 1: 16 slots further
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t n = wcol(ct);
            const int64_t gs = g / gm;
            sdst[ct] = sc[gs * N + n];
            zdst[ct] = ZERO ? zp[(gs * N + n) >> 1] : (uint8_t)0;
        }
    };

    f32x16_t yacc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[rt][ct][r] = 0.f;

    load_x(0);
    load_b(0, braw, sraw, zraw);
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
    auto step = [&](int g, const u32x4_t (&bw)[CT][2], const uint16_t (&sw)[CT], const uint8_t (&zw)[CT],
                    u32x4_t (&bn)[CT][2], uint16_t (&sn)[CT], uint8_t (&zn)[CT]) {
        const int buf = g & 1;
        const int gn = g + 1 < G ? g + 1 : g;
        load_x(gn);
        load_b(gn, bn, sn, zn);
        float s[CT];
        uint32_t nb2[CT];
        u32x4_t bcorr[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int64_t n = wcol(ct);
            s[ct] = h2f<DT>(sw[ct]);
            uint32_t z = 8;
            if constexpr (ZERO) z = __builtin_amdgcn_ubfe((uint32_t)zw[ct], (uint32_t)(n & 1) * 4u, 4);
            if constexpr (CORR) {
                const uint32_t c = bf16_negbias(z);
                bcorr[ct] = kg == 0 ? u32x4_t{c | (c << 16), c, 0, 0} : u32x4_t{0, 0, 0, 0};
                nb2[ct] = 0;
            } else {
                nb2[ct] = f16_negbias2(z);
            }
        }
        const uint8_t *abase = lds + buf * BM * ROWB + arow * ROWB + kg * 128;
        // accumulator inputs of the first step: the bias correction (bf16; one
        // per row tile when every column has z = 8, else one per column tile)
        // or zero.  Passing it as the matrix-core C input avoids copying one
        // correction into several accumulators.
        f32x16_t cin[RT][ZERO ? CT : 1];
        if constexpr (CORR) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t *>(
                    lds + buf * BM * ROWB + (arow + rt * 32) * ROWB + 256 + kg * 16);
#pragma unroll
                for (int ci = 0; ci < (ZERO ? CT : 1); ++ci) cin[rt][ci] = mfma32x32x16<DT>(a, bcorr[ci], f32x16_t{});
            }
        }
        f32x16_t acc[RT][CT];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            u32x4_t a[RT], bq[CT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                a[rt] = *reinterpret_cast<const u32x4_t *>(abase + rt * 32 * ROWB + t * 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) bq[ct] = dequant_word<DT>(bw[ct][t >> 2][t & 3], nb2[ct]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if (t == 0) {
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
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 16; ++r) yacc[rt][ct][r] += s[ct] * acc[rt][ct][r];
        __syncthreads();
    };
    for (int g = 0; g < G; g += 2) {
        step(g, braw, sraw, zraw, bnext, snext, znext);
        if (g + 1 < G) step(g + 1, bnext, snext, znext, braw, sraw, zraw);
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
static int g_tile_cfg = -1;      // -1: automatic

int tile_config_count() { return (int)(sizeof(kTileCfgs) / sizeof(kTileCfgs[0])); }
void set_tile_config(int idx) { g_tile_cfg = idx; }

template <int DT, bool ZERO, bool GROUPED, int BM, int BN, int WM, int WN, bool SILU = false>
static hipError_t tile_launch(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                              const void *scale, const void *zero, void *y, int64_t M, int64_t K, int64_t N,
                              int64_t E, int gm, const float *cs, const float *cz, hipStream_t stream) {
    // grouped: every expert may end in a partial row tile, hence + E; the
    // items go on a 1-D grid rounded up to whole rounds over the XCDs
    const int64_t ncb = SILU ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
    const int64_t mtiles = GROUPED ? (M + BM - 1) / BM + E : (M + BM - 1) / BM;
    const int64_t slots = (mtiles * ncb + kXcds - 1) / kXcds * kXcds;
    if (GROUPED && slots > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid = GROUPED ? dim3((unsigned)slots) : dim3((unsigned)mtiles, (unsigned)ncb);
    hipLaunchKernelGGL((gemm_tile_kernel<DT, ZERO, BM, BN, WM, WN, GROUPED, SILU>), grid, dim3(WM * WN * 64), 0,
                       stream, (const uint16_t *)x, offsets, row_src, (const uint8_t *)wp, (const uint16_t *)scale,
                       (const uint8_t *)zero, (uint16_t *)y, M, K, N, (int)E, gm, cs, cz);
    return hipGetLastError();
}

template <int DT, bool ZERO, bool GROUPED>
static hipError_t tile_dispatch(const void *x, const int32_t *offsets, const int32_t *row_src, const void *wp,
                                const void *scale, const void *zero, void *y, int64_t M, int64_t K, int64_t N,
                                int64_t E, int gm, const float *cs, const float *cz, hipStream_t stream) {
    int idx = g_tile_cfg;
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
    int idx = g_tile_cfg;
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

hipError_t launch_gemm_tile(const void *x, const int32_t *offsets, const void *wp, const void *scale,
                            const void *zero, void *y, int64_t M, int64_t K, int64_t N, int64_t E,
                            int dt, hipStream_t stream, const int32_t *row_src, int gm, const float *cs,
                            const float *cz) {
    if (offsets) return tile_dispatch_dt<true>(x, offsets, row_src, wp, scale, zero, y, M, K, N, E, gm, dt, cs, cz, stream);
    return tile_dispatch_dt<false>(x, nullptr, row_src, wp, scale, zero, y, M, K, N, 1, gm, dt, cs, cz, stream);
}

}  // namespace w4
