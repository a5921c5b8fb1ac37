// common.hpp — device helpers shared by the libw4a16 kernels (gfx950 only).
//
// Prepacked weight tile (see include/w4a16.h): 1024 bytes per (16-column
// block, 128-row group).  Slot L = 16*c + j (c = 32-row chunk 0..3, j =
// column 0..15) is 16 bytes = 4 words; word t holds rows r = 32c + 8t + i,
// i = 0..7, with the code of row r at bit 4*(i/2) + 16*(i%2).  One 128-bit
// load therefore gives a lane the 32 codes of one column for one chunk, and
//   ((word >> 4p) & 0x000F000F)
// is the pair (i = 2p, i = 2p+1) already in the low/high 16-bit halves that
// the 16-bit matrix-core operand register expects.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8_t __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2_t __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef int i32x4_t __attribute__((__vector_size__(4 * sizeof(int))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

enum { DT_F16 = 0, DT_BF16 = 1 };

typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

// Reinterpret a 32-bit value.  Takes the word BY VALUE on purpose: this
// compiler lowers __builtin_bit_cast applied directly to a vector-subscript
// expression (v[i]) as a read of element 0, so vector elements must pass
// through a scalar first.
template <typename T>
__device__ __forceinline__ T as(uint32_t w) { return __builtin_bit_cast(T, w); }

constexpr int kGroup = 128;          // K rows per quantization group
constexpr int kTileBytes = 1024;     // one (16-column, 128-row) weight tile

// ---------------------------------------------------------------------------
// 16-bit float <-> fp32
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float h2f(uint16_t b) {
    if constexpr (DT == DT_BF16) {
        return __uint_as_float(((uint32_t)b) << 16);
    } else {
        _Float16 h = __builtin_bit_cast(_Float16, b);
        return (float)h;
    }
}

// Round-to-nearest-even fp32 -> 16-bit pattern.
template <int DT>
__device__ __forceinline__ uint16_t f2h(float v) {
    if constexpr (DT == DT_BF16) {
        __bf16 b = (__bf16)v;          // v_cvt_pk_bf16_f32: RNE
        return __builtin_bit_cast(uint16_t, b);
    } else {
        _Float16 h = (_Float16)v;      // v_cvt_f16_f32: RNE
        return __builtin_bit_cast(uint16_t, h);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core wrappers.  Operands are passed as four 32-bit registers.
//
// The destination of a matrix-core instruction must not share registers with
// its A or B operand: the result registers are written while later passes
// still read the sources.  The register allocator does not enforce this when
// A/B die at the instruction (it happily reuses them for the result when the
// accumulator input is a constant), so every wrapper keeps A and B alive
// until after the instruction with an empty asm use (no code is emitted).
// ---------------------------------------------------------------------------
template <typename R, typename A, typename B>
__device__ __forceinline__ void keep_live(R &r, const A &a, const B &b) {
    asm volatile("" : "+v"(r) : "v"(a), "v"(b));
}
template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
    f32x4_t r;
    if constexpr (DT == DT_BF16)
        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    keep_live(r, a, b);
    return r;
}

template <int DT>
__device__ __forceinline__ f32x16_t mfma32x32x16(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
    f32x16_t r;
    if constexpr (DT == DT_BF16)
        r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        r = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    keep_live(r, a, b);
    return r;
}

typedef short s16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// 16x16x16 bf16 step with 2-register operands (4 bf16 per lane: lane l feeds
// row/column l % 16, k-block l / 16; result layout as for 16x16x32).
__device__ __forceinline__ f32x4_t mfma16x16x16_bf16(const u32x2_t &a, const u32x2_t &b, const f32x4_t &c) {
    f32x4_t r = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                                __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
    keep_live(r, a, b);
    return r;
}

__device__ __forceinline__ i32x4_t mfma_i8_16x16x64(const u32x4_t &a, const u32x4_t &b, const i32x4_t &c) {
    i32x4_t r = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                                            __builtin_bit_cast(i32x4_t, b), c, 0, 0, 0);
    keep_live(r, a, b);
    return r;
}

// ---------------------------------------------------------------------------
// In-register dequantization of one prepacked word (8 codes) into the 16-bit
// operand of one 16-k matrix-core step.
//
// bf16: a 16-bit pattern with high byte 0x43 and the code in the low byte is
//       exactly 128 + v (exponent of 128, code in the 7 mantissa bits).  The
//       bias (128 + z) is removed inside the matrix core by an extra
//       correction step (see the kernels).
// fp16: high byte 0x64 and the code in the low byte is 1024 + v; one packed
//       fp16 add of -(1024 + z) gives the exact integer v - z.
// ---------------------------------------------------------------------------

// One prepacked word holds rows i = 0..7 of a chunk at bit 4*(i/2) + 16*(i%2),
// so lo = word & 0x0F0F0F0F has rows (0, 4, 1, 5) in its bytes and
// hi = (word >> 4) & 0x0F0F0F0F has rows (2, 6, 3, 7).  Each operand register
// (rows 2p, 2p+1 in its low/high 16 bits) is then one v_perm_b32 that places
// a code byte under the exponent byte of the magic number: 7 vector ALU
// instructions per 8 weights, all visible to the compiler's hazard tracking.
template <int DT>
__device__ __forceinline__ u32x4_t dequant_word(uint32_t w, uint32_t negbias2) {
    constexpr uint32_t expb = DT == DT_BF16 ? 0x43434343u : 0x64646464u;   // exponent byte of 128 / 1024
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    u32x4_t r;
    // v_perm_b32 selector bytes: 0-3 pick bytes of the second source, 4-7 of the first
    r[0] = __builtin_amdgcn_perm(expb, lo, 0x04020400u);   // rows 0, 1
    r[1] = __builtin_amdgcn_perm(expb, hi, 0x04020400u);   // rows 2, 3
    r[2] = __builtin_amdgcn_perm(expb, lo, 0x04030401u);   // rows 4, 5
    r[3] = __builtin_amdgcn_perm(expb, hi, 0x04030401u);   // rows 6, 7
    if constexpr (DT == DT_F16) {
        const f16x2_t nb = as<f16x2_t>(negbias2);
#pragma unroll
        for (int p = 0; p < 4; ++p) r[p] = __builtin_bit_cast(uint32_t, as<f16x2_t>(r[p]) + nb);
    } else {
        (void)negbias2;
    }
    return r;
}

// -(1024 + z) as an fp16 pair (exact: 1024 + z < 2048).
__device__ __forceinline__ uint32_t f16_negbias2(uint32_t z) {
    uint32_t h = 0xE400u + z;     // fp16 bits of -(1024 + z)
    return h | (h << 16);
}

// -(128 + z) as bf16 bits (exact: 128 + z < 256 has 8 significant bits).
__device__ __forceinline__ uint32_t bf16_negbias(uint32_t z) { return 0xC300u + z; }

// bf16 RNE of an fp32 value, returned as raw bits, and its exact fp32 value.
__device__ __forceinline__ uint32_t bf16_bits_rne(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Split an fp32 value into three bf16 limbs hi + mid + lo (24 significant
// bits in total; each subtraction is exact).
__device__ __forceinline__ void split3_bf16(float v, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
    hi = bf16_bits_rne(v);
    float r1 = v - __uint_as_float(hi << 16);
    mid = bf16_bits_rne(r1);
    float r2 = r1 - __uint_as_float(mid << 16);
    lo = bf16_bits_rne(r2);
}

// Signed int8 operand from biased 4-bit codes (q + 8 in 0..15) held in the
// low nibble of each byte: (b + 0x78) ^ 0x80 = q as two's complement, with no
// carry between bytes (b + 0x78 <= 0x87).
__device__ __forceinline__ uint32_t codes_to_s8(uint32_t b) { return (b + 0x78787878u) ^ 0x80808080u; }

__device__ __forceinline__ u32x4_t ld128(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the 64 lanes of a wave (every lane active): DPP
// shifts by 1, 2, 4 and 8 lanes within each 16-lane row (lanes shifted in
// from outside the row add 0), then the rows' totals are added by the
// broadcasts of lanes 15 and 31.  No LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
    return v;
}

}  // namespace w4
