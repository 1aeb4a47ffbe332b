// Device helpers shared by the LoRA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// Two float32 values -> packed bf16 pair (round to nearest even; low half = lo).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// One 16x16x32 bf16 MFMA: acc[16x16] += a[16x32] * b[32x16].
// Operand lane layout: lane l supplies row (a) / column (b) l % 16 and one
// 8-element slice of the 32-long contraction selected by l / 16; the two
// operands use the same slice mapping.  Result: lane l holds rows
// 4*(l/16) + {0,1,2,3} of column l % 16.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
    return __builtin_bit_cast(bf16x8, v);
}

// Workgroup -> tile index such that the tiles one XCD runs are contiguous.
// Workgroups are dispatched to the 8 XCDs round-robin (wg % 8); this gives
// XCD x the contiguous range of tile ids [start_x, start_x + count_x).
__device__ __forceinline__ int xcd_contiguous(int bid, int total) {
    const int per = total >> 3, rem = total & 7;
    const int x = bid & 7, i = bid >> 3;
    return x * per + min(x, rem) + i;
}

// Tile id -> (row tile, col tile) in groups of G row tiles, column-major inside
// a group, so consecutive ids share a few row panels and column panels.
template <int G>
__device__ __forceinline__ void grouped_tile(int t, int n_row, int n_col, int& rt, int& ct) {
    const int per_group = G * n_col;
    const int g = t / per_group;
    const int first = g * G;
    const int gs = min(n_row - first, G);
    const int idx = t - g * per_group;
    rt = first + idx % gs;
    ct = idx / gs;
}

}  // namespace lora
