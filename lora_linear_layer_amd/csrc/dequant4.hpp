// Standalone 4-bit weight dequantisation (page "Unsloth — 微调 2-5x 加速",
// section "核心要点", item 3: 4-bit frozen weights restored for the matmul).
// Format: codes [N][K/2] (element k in the low nibble of byte k/2 when k is
// even, the high nibble when odd), one fp16 absmax per 64 consecutive k, a
// 16-entry float32 codebook.  Value = codebook[code] * float32(absmax) in
// float32, then rounded to bf16 for a bf16 output.  HBM-bound.
#pragma once
#include "common.hpp"

namespace lora {

// Standalone 4-bit dequantisation: W_out[n][k] for 16 consecutive k per thread.
template <bool F32_OUT>
__global__ __launch_bounds__(256) void dequant4_kernel(const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ absmax,
                                                      const float* __restrict__ codebook, void* __restrict__ out,
                                                      int64_t N, int64_t K) {
    __shared__ f32x2 lut[256];
    const int tid = threadIdx.x;
    lut[tid] = f32x2{codebook[tid & 15], codebook[tid >> 4]};
    __syncthreads();
    const int64_t groups_per_row = K / 16;
    const int64_t gid = (int64_t)blockIdx.x * 256 + tid;
    if (gid >= N * groups_per_row) return;
    const int64_t n = gid / groups_per_row;
    const int64_t k = (gid - n * groups_per_row) * 16;
    const u32x2 codes = *reinterpret_cast<const u32x2*>(Wq + n * (K / 2) + k / 2);
    const float am = f16_bits_to_f32(absmax[n * (K / 64) + k / 64]);
    float v[16];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint32_t byte = (codes[b >> 2] >> (8 * (b & 3))) & 0xFFu;
        const f32x2 e = lut[byte];
        v[2 * b] = e[0] * am;
        v[2 * b + 1] = e[1] * am;
    }
    if constexpr (F32_OUT) {
        f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + n * K + k);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    } else {
        u32x4* o = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + n * K + k);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            o[i] = u32x4{pack_bf16x2(v[8 * i], v[8 * i + 1]), pack_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                         pack_bf16x2(v[8 * i + 4], v[8 * i + 5]), pack_bf16x2(v[8 * i + 6], v[8 * i + 7])};
    }
}

}  // namespace lora
