// RMSNorm in front of the LoRA linear (page "ms-swift框架下UnSloth与Liger-Kernel
// 优化实战", section "关键融合策略解析", RMSNorm + Linear: the normalised
// activations are not written out and read back by the linear).
//
//   Xn[m][k] = X[m][k] * inv[m] * g[k],   inv[m] = 1 / sqrt(mean_k X[m][k]^2 + eps)
//
// The norm weight g is frozen (part of the backbone, like W), so it is folded
// once into the frozen weight, W_g = W diag(g) (lora_fold_norm_weight), and per
// call into A (A_g = A diag(g), r x K).  The GEMMs then read the raw X and
// apply inv[m] to each output row in the epilogue:
//   H = inv (X W_g^T + s (X A_g^T) B^T),  U = inv X A_g^T.
// The input gradient through the norm, with D = dY W_g + s V A_g (= g dXn,
// the plain dX GEMM with the folded operands):
//   dX = inv D - X (inv^3 / K) <D, X>_row
// (from dx = inv g dxn - x inv^3 / K sum_k g_k dxn_k x_k).  These are the
// memory-bound row kernels of that path.
#pragma once
#include "common.hpp"

namespace lora {

// Sum over a wave (64 lanes) with cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// inv[m] = 1 / sqrt(mean_k X[m][k]^2 + eps): one wave per row (K % 8 == 0),
// 16-byte loads, float32 sums.
__global__ __launch_bounds__(256) void rms_inv_kernel(const uint16_t* __restrict__ X, float* __restrict__ inv,
                                                      int M, int K, float eps) {
    const int lane = threadIdx.x & 63;
    const int m = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint16_t* row = X + (size_t)m * K;
    float ss = 0.f;
    for (int c = lane * 8; c < K; c += 64 * 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16_bits_to_f32(v[i] & 0xFFFFu), hi = bf16_bits_to_f32(v[i] >> 16);
            ss += lo * lo + hi * hi;
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) inv[m] = 1.0f / sqrtf(ss / (float)K + eps);
}

// out[i][k] = bf16(in[i][k] * g[k]) for R rows of K columns (K % 8 == 0): the
// norm weight folded into W (once) or A (per call).  out may be in: each
// thread reads its 8 elements before it writes them.
__global__ __launch_bounds__(256) void scale_cols_kernel(const uint16_t* in, const uint16_t* __restrict__ g,
                                                         uint16_t* out, int64_t R, int K) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;     // 8 consecutive elements
    if (e >= R * K) return;
    const int k = (int)(e % K);
    const u32x4 v = *reinterpret_cast<const u32x4*>(in + e);
    const u32x4 w = *reinterpret_cast<const u32x4*>(g + k);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = bf16_bits_to_f32(v[i] & 0xFFFFu) * bf16_bits_to_f32(w[i] & 0xFFFFu);
        const float hi = bf16_bits_to_f32(v[i] >> 16) * bf16_bits_to_f32(w[i] >> 16);
        o[i] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(out + e) = o;
}

// The norm's input gradient, in place: dX[m][k] = inv[m] D[m][k] - X[m][k] c[m]
// with c[m] = inv[m]^3 / K sum_k D[m][k] X[m][k]; D arrives in dX (bf16).  One
// wave per row: the row's dot product, then the update (the row's second
// read is served by the caches).
__global__ __launch_bounds__(256) void norm_dx_kernel(uint16_t* __restrict__ dX, const uint16_t* __restrict__ X,
                                                      const float* __restrict__ inv, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int m = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    uint16_t* drow = dX + (size_t)m * K;
    const uint16_t* xrow = X + (size_t)m * K;
    float dot = 0.f;
    for (int c = lane * 8; c < K; c += 64 * 8) {
        const u32x4 d = *reinterpret_cast<const u32x4*>(drow + c);
        const u32x4 x = *reinterpret_cast<const u32x4*>(xrow + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dot += bf16_bits_to_f32(d[i] & 0xFFFFu) * bf16_bits_to_f32(x[i] & 0xFFFFu);
            dot += bf16_bits_to_f32(d[i] >> 16) * bf16_bits_to_f32(x[i] >> 16);
        }
    }
    dot = wave_sum(dot);
    const float iv = inv[m];
    const float cm = iv * iv * iv / (float)K * dot;
    for (int c = lane * 8; c < K; c += 64 * 8) {
        const u32x4 d = *reinterpret_cast<const u32x4*>(drow + c);
        const u32x4 x = *reinterpret_cast<const u32x4*>(xrow + c);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = iv * bf16_bits_to_f32(d[i] & 0xFFFFu) - bf16_bits_to_f32(x[i] & 0xFFFFu) * cm;
            const float hi = iv * bf16_bits_to_f32(d[i] >> 16) - bf16_bits_to_f32(x[i] >> 16) * cm;
            o[i] = pack_bf16x2(lo, hi);
        }
        *reinterpret_cast<u32x4*>(drow + c) = o;
    }
}

}  // namespace lora
