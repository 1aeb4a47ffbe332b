// Standalone 4-bit weight dequantisation (page "Unsloth — 微调 2-5x 加速",
// section "核心要点", item 3: 4-bit frozen weights restored for the matmul).
// Format: codes [N][K/2] (element k in the low nibble of byte k/2 when k is
// even, the high nibble when odd), one fp16 absmax per 64 consecutive k, a
// 16-entry float32 codebook.  Value = codebook[code] * float32(absmax) in
// float32, then rounded to bf16 for a bf16 output.  HBM-bound.
#pragma once
#include "common.hpp"
#include "stream_store.hpp"

namespace lora {

// Standalone 4-bit dequantisation over the flat index e = n K + k (K % 64 == 0,
// so code byte e / 2, absmax entry e / 64 and output element e line up without
// row arithmetic; N K < 2^31, checked by the caller).  A group is 8 consecutive
// weights: one 4-byte code load, one absmax, one 16-byte (bf16) or two (float32)
// stores, so each wave instruction touches one contiguous range.  The grid
// strides over the groups, four per thread per iteration to keep loads in
// flight; the 256-entry byte -> (low, high) codebook table is built in LDS once
// per workgroup.
template <bool F32_OUT>
__global__ __launch_bounds__(256) void dequant4_kernel(const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ absmax,
                                                      const float* __restrict__ codebook, void* __restrict__ out,
                                                      int n_groups) {
    __shared__ f32x2 lut[256];
    const int tid = threadIdx.x;
    lut[tid] = f32x2{codebook[tid & 15], codebook[tid >> 4]};
    __syncthreads();
    const uint32_t* const cw = reinterpret_cast<const uint32_t*>(Wq);
    const int stride = (int)gridDim.x * 256;
    auto emit = [&](int g, uint32_t codes, float am) {
        float v[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x2 e = lut[(codes >> (8 * b)) & 0xFFu];
            v[2 * b] = e[0] * am;
            v[2 * b + 1] = e[1] * am;
        }
        if constexpr (F32_OUT) {
            f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)g * 8);
            store_stream(o, f32x4{v[0], v[1], v[2], v[3]});
            store_stream(o + 1, f32x4{v[4], v[5], v[6], v[7]});
        } else {
            store_stream(reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (size_t)g * 8),
                         u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7])});
        }
    };
    int g = (int)blockIdx.x * 256 + tid;
    for (; g + 3 * stride < n_groups; g += 4 * stride) {
        uint32_t c[4];
        float am[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = cw[g + i * stride];
            am[i] = f16_bits_to_f32(absmax[(g + i * stride) >> 3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) emit(g + i * stride, c[i], am[i]);
    }
    for (; g < n_groups; g += stride) emit(g, cw[g], f16_bits_to_f32(absmax[g >> 3]));
}

}  // namespace lora
