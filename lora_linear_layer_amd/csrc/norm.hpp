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

constexpr int kRowChunk = 64 * 8;      // elements one wave covers with one 16-byte load per lane

__device__ __forceinline__ float dot_bf16x8(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc += bf16_bits_to_f32(a[i] & 0xFFFFu) * bf16_bits_to_f32(b[i] & 0xFFFFu);
        acc += bf16_bits_to_f32(a[i] >> 16) * bf16_bits_to_f32(b[i] >> 16);
    }
    return acc;
}

// Sum of squares of one bf16 row of K elements (K % 8 == 0) over one wave,
// NV 16-byte loads per lane issued together (the row's bytes in flight at once).
template <int NV>
__device__ __forceinline__ float row_sumsq(const uint16_t* row, int K, int lane) {
    float ss = 0.f;
    for (int c0 = lane * 8; c0 < K; c0 += kRowChunk * NV) {
        u32x4 v[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int c = c0 + u * kRowChunk;
            v[u] = c < K ? *reinterpret_cast<const u32x4*>(row + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) ss = dot_bf16x8(v[u], v[u], ss);
    }
    return wave_sum(ss);
}

// The norm's per-call preparation, one launch: blocks [0, rms_blocks) write
// inv[m] = 1 / sqrt(mean_k X[m][k]^2 + eps) (one wave per row, four rows per
// block; skipped when rms_blocks = 0); the rest write out[i][k] = bf16(in[i][k]
// g[k]) for R rows of K columns, 8 elements per thread (A diag(g), or W diag(g)
// when the weight is folded).  out may be in: each thread reads its 8
// elements before it writes them.
struct NormPrepArgs {
    const uint16_t* X;
    float* inv;
    int M, K, rms_blocks;
    float eps;
    const uint16_t* in;
    const uint16_t* g;
    uint16_t* out;
    int64_t R;
};

__global__ __launch_bounds__(256) void norm_prep_kernel(const NormPrepArgs a) {
    if ((int)blockIdx.x < a.rms_blocks) {
        const int lane = threadIdx.x & 63;
        const int m = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
        if (m >= a.M) return;
        const float ss = row_sumsq<8>(a.X + (size_t)m * a.K, a.K, lane);
        if (lane == 0) a.inv[m] = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        return;
    }
    const int64_t e = ((int64_t)(blockIdx.x - a.rms_blocks) * 256 + threadIdx.x) * 8;
    if (e >= a.R * a.K) return;
    const int k = (int)(e % a.K);
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.in + e);
    const u32x4 w = *reinterpret_cast<const u32x4*>(a.g + k);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = bf16_bits_to_f32(v[i] & 0xFFFFu) * bf16_bits_to_f32(w[i] & 0xFFFFu);
        const float hi = bf16_bits_to_f32(v[i] >> 16) * bf16_bits_to_f32(w[i] >> 16);
        o[i] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(a.out + e) = o;
}

// The norm's input gradient, in place: dX[m][k] = inv[m] D[m][k] - X[m][k] c[m]
// with c[m] = inv[m]^3 / K sum_k D[m][k] X[m][k]; D arrives in dX (bf16).  One
// wave per row.  NV > 0 (K <= NV * 512): the row of D and of X is loaded once
// into registers, all loads issued together, then the dot product and the
// update.  NV = 0: any K, two streamed passes (the second read served by the
// caches).
__device__ __forceinline__ u32x4 norm_dx_apply(u32x4 d, u32x4 x, float iv, float cm) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = iv * bf16_bits_to_f32(d[i] & 0xFFFFu) - bf16_bits_to_f32(x[i] & 0xFFFFu) * cm;
        const float hi = iv * bf16_bits_to_f32(d[i] >> 16) - bf16_bits_to_f32(x[i] >> 16) * cm;
        o[i] = pack_bf16x2(lo, hi);
    }
    return o;
}

template <int NV>
__global__ __launch_bounds__(256) void norm_dx_kernel(uint16_t* __restrict__ dX, const uint16_t* __restrict__ X,
                                                      const float* __restrict__ inv, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int m = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    uint16_t* drow = dX + (size_t)m * K;
    const uint16_t* xrow = X + (size_t)m * K;
    const float iv = inv[m];
    if constexpr (NV > 0) {
        u32x4 d[NV], x[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int c = lane * 8 + u * kRowChunk;
            d[u] = c < K ? *reinterpret_cast<const u32x4*>(drow + c) : u32x4{0u, 0u, 0u, 0u};
            x[u] = c < K ? *reinterpret_cast<const u32x4*>(xrow + c) : u32x4{0u, 0u, 0u, 0u};
        }
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < NV; ++u) dot = dot_bf16x8(d[u], x[u], dot);
        dot = wave_sum(dot);
        const float cm = iv * iv * iv / (float)K * dot;
        // keep the row packed between the two uses: without this the compiler
        // holds all its float32 conversions live and the kernel spills
#pragma unroll
        for (int u = 0; u < NV; ++u) asm volatile("" : "+v"(d[u]), "+v"(x[u]));
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int c = lane * 8 + u * kRowChunk;
            if (c < K) *reinterpret_cast<u32x4*>(drow + c) = norm_dx_apply(d[u], x[u], iv, cm);
        }
    } else {
        constexpr int U = 4;
        float dot = 0.f;
        for (int c0 = lane * 8; c0 < K; c0 += kRowChunk * U) {
            u32x4 d[U], x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kRowChunk;
                d[u] = c < K ? *reinterpret_cast<const u32x4*>(drow + c) : u32x4{0u, 0u, 0u, 0u};
                x[u] = c < K ? *reinterpret_cast<const u32x4*>(xrow + c) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) dot = dot_bf16x8(d[u], x[u], dot);
        }
        dot = wave_sum(dot);
        const float cm = iv * iv * iv / (float)K * dot;
        for (int c = lane * 8; c < K; c += kRowChunk) {
            const u32x4 d = *reinterpret_cast<const u32x4*>(drow + c);
            const u32x4 x = *reinterpret_cast<const u32x4*>(xrow + c);
            *reinterpret_cast<u32x4*>(drow + c) = norm_dx_apply(d, x, iv, cm);
        }
    }
}

}  // namespace lora
