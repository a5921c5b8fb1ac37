// prepack.hip — offline weight repack into the tile layout, and its inverse.
//
// One 64-thread workgroup per 1024-byte tile (expert e, 16-column block nb,
// 128-row group g).  The tile's source region (128 rows x 8 bytes of the plain
// [K][N/2] layout) is staged in LDS, then each lane assembles its 16-byte slot.
// The reorder follows the "Marlin layout" idea (pwwt.cn notes §6.2: weights
// reordered for memory access, kernels matched to the layout) and QUICK's
// offline interleave (weights laid out so the dequantized values go straight
// into the matrix-multiply operand without a shared-memory write-back).
//
// Layout 1 (group-aligned, for scale groups of 32 or 64 rows) exchanges the
// roles of the slot's chunk c = L / 16 and the word t: word t of slot L holds
// rows 128*g + 32*t + 8*c + i instead of 128*g + 32*c + 8*t + i, so the 32
// rows one 16x16x32 matrix-core step takes from the four chunks (one word of
// each lane) are the consecutive rows 32*t .. 32*t + 31 of one scale group.
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

__device__ __forceinline__ int code_shift(int i) { return 4 * (i >> 1) + 16 * (i & 1); }

// row of the 128-row block held by word t, code i of chunk c's slots
__device__ __forceinline__ int slot_row(int layout, int c, int t, int i) {
    return layout == 1 ? 32 * t + 8 * c + i : 32 * c + 8 * t + i;
}

__global__ void __launch_bounds__(64) prepack_kernel(const uint8_t *__restrict__ w, uint8_t *__restrict__ out,
                                                     int64_t K, int64_t N, int is_signed, int layout) {
    const int64_t G = K / kGroup, NB = N / 16;
    const int64_t tile = blockIdx.x;                 // (e * NB + nb) * G + g
    const int64_t g = tile % G;
    const int64_t nb = (tile / G) % NB;
    const int64_t e = tile / (G * NB);
    const int L = threadIdx.x;

    __shared__ uint64_t rows[kGroup];                 // 16 codes of each row
    const uint8_t *src = w + e * K * (N / 2) + (g * kGroup) * (N / 2) + nb * 8;
    for (int r = L; r < kGroup; r += 64)
        rows[r] = *reinterpret_cast<const uint64_t *>(src + (int64_t)r * (N / 2));
    __syncthreads();

    const int c = L >> 4, j = L & 15;
    u32x4_t slot;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t code = (uint32_t)(rows[slot_row(layout, c, t, i)] >> (4 * j)) & 0xFu;
            if (is_signed) code ^= 0x8u;              // q + 8 for two's complement q
            word |= code << code_shift(i);
        }
        slot[t] = word;
    }
    *reinterpret_cast<u32x4_t *>(out + tile * kTileBytes + L * 16) = slot;
}

__global__ void __launch_bounds__(64) unpack_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ w,
                                                    int64_t K, int64_t N, int is_signed, int layout) {
    const int64_t G = K / kGroup, NB = N / 16;
    const int64_t tile = blockIdx.x;
    const int64_t g = tile % G;
    const int64_t nb = (tile / G) % NB;
    const int64_t e = tile / (G * NB);
    const int L = threadIdx.x;

    __shared__ uint32_t words[256];
    const u32x4_t s = ld128(in + tile * kTileBytes + L * 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) words[4 * L + t] = s[t];
    __syncthreads();

    uint8_t *dst = w + e * K * (N / 2) + (g * kGroup) * (N / 2) + nb * 8;
    for (int r = L; r < kGroup; r += 64) {
        const int c = layout == 1 ? (r >> 3) & 3 : r >> 5;
        const int t = layout == 1 ? r >> 5 : (r >> 3) & 3;
        const int i = r & 7;
        uint64_t row = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t code = (words[4 * (16 * c + j) + t] >> code_shift(i)) & 0xFu;
            if (is_signed) code ^= 0x8u;
            row |= (uint64_t)code << (4 * j);
        }
        *reinterpret_cast<uint64_t *>(dst + (int64_t)r * (N / 2)) = row;
    }
}

hipError_t launch_prepack(const void *w, void *out, int64_t E, int64_t K, int64_t N, int is_signed,
                          hipStream_t stream, int layout) {
    const int64_t tiles = E * (N / 16) * (K / kGroup);
    hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)tiles), dim3(64), 0, stream,
                       (const uint8_t *)w, (uint8_t *)out, K, N, is_signed, layout);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *in, void *w, int64_t E, int64_t K, int64_t N, int is_signed,
                         hipStream_t stream, int layout) {
    const int64_t tiles = E * (N / 16) * (K / kGroup);
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)tiles), dim3(64), 0, stream,
                       (const uint8_t *)in, (uint8_t *)w, K, N, is_signed, layout);
    return hipGetLastError();
}

}  // namespace w4
