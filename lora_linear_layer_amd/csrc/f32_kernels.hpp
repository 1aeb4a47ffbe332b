// Float32 checking mode: the same layer in plain float32 SIMT arithmetic
// (no bf16 rounding anywhere).  Correctness-first; not a performance path.
//   Z[p][j]   = sum_c Y[p][c] F(j, c)                       (f32_skinny)
//   Out[p][q] = sum_c L[p][c] R(q, c) + s sum_j E(q, j) Z[p][j]   (f32_fused)
//   G[c][j]   = sum_m Y[m][c] Z[m][j], scaled by s          (f32_grad)
// Role mapping is the same as in the bf16 GEMM (lora_gemm.hpp).
#pragma once
#include "common.hpp"

namespace lora {

enum F32RMode { kRDirect = 0, kRTrans = 1, kRQuantDirect = 2, kRQuantTrans = 3 };

struct F32FusedArgs {
    const float* L;         // [P][C]
    const float* R;         // kRDirect: [Q][C]; kRTrans: [C][Q]
    const uint8_t* Rq;      // quant: codes, [Q][C/2] or [C][Q/2]
    const uint16_t* Rabs;   // quant: fp16 absmax, [Q][C/64] or [C][Q/64]
    const float* codebook;
    const float* E;         // e_trans = 0: [Q][r]; 1: [r][Q]
    const float* Z;         // [P][r]
    float* Out;             // [P][Q]
    int P, Q, C, r, e_trans;
    float s;
};

template <int RMODE>
__device__ __forceinline__ float f32_r_at(const F32FusedArgs& a, int q, int c) {
    if constexpr (RMODE == kRDirect) return a.R[(size_t)q * a.C + c];
    if constexpr (RMODE == kRTrans) return a.R[(size_t)c * a.Q + q];
    if constexpr (RMODE == kRQuantDirect) {
        const uint8_t byte = a.Rq[(size_t)q * (a.C >> 1) + (c >> 1)];
        const int code = (c & 1) ? (byte >> 4) : (byte & 15);
        return a.codebook[code] * f16_bits_to_f32(a.Rabs[(size_t)q * (a.C >> 6) + (c >> 6)]);
    }
    // kRQuantTrans: the weight is stored [C][Q] (rows c, 4-bit along q)
    const uint8_t byte = a.Rq[(size_t)c * (a.Q >> 1) + (q >> 1)];
    const int code = (q & 1) ? (byte >> 4) : (byte & 15);
    return a.codebook[code] * f16_bits_to_f32(a.Rabs[(size_t)c * (a.Q >> 6) + (q >> 6)]);
}

template <int RMODE>
__global__ __launch_bounds__(256) void f32_fused(const F32FusedArgs a) {
    __shared__ float Ls[16][65];
    __shared__ float Rs[16][65];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int p0 = blockIdx.y * 64, q0 = blockIdx.x * 64;
    float acc[4][4] = {};
    for (int c0 = 0; c0 < a.C; c0 += 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;       // 1024 elements: 64 rows x 16 c
            const int row = e >> 4, cl = e & 15;
            const int c = c0 + cl;
            const int p = p0 + row, q = q0 + row;
            Ls[cl][row] = (p < a.P && c < a.C) ? a.L[(size_t)p * a.C + c] : 0.f;
            Rs[cl][row] = (q < a.Q && c < a.C) ? f32_r_at<RMODE>(a, q, c) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int cl = 0; cl < 16; ++cl) {
            float lv[4], rv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { lv[i] = Ls[cl][ty * 4 + i]; rv[i] = Rs[cl][tx * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += lv[i] * rv[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = p0 + ty * 4 + i;
        if (p >= a.P) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = q0 + tx * 4 + j;
            if (q >= a.Q) continue;
            float lo = 0.f;
            for (int jj = 0; jj < a.r; ++jj) {
                const float e = a.e_trans ? a.E[(size_t)jj * a.Q + q] : a.E[(size_t)q * a.r + jj];
                lo += e * a.Z[(size_t)p * a.r + jj];
            }
            a.Out[(size_t)p * a.Q + q] = acc[i][j] + a.s * lo;
        }
    }
}

// Z[p][j] = sum_c Y[p][c] F(j, c); f_trans = 0: F = [r][C]; 1: F(j, c) = F[c][j].
__global__ __launch_bounds__(256) void f32_skinny(const float* __restrict__ Y, const float* __restrict__ F,
                                                 float* __restrict__ Z, int P, int C, int r, int f_trans) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)P * r) return;
    const int p = (int)(e / r), j = (int)(e % r);
    float sum = 0.f;
    for (int c = 0; c < C; ++c) {
        const float f = f_trans ? F[(size_t)c * r + j] : F[(size_t)j * C + c];
        sum += Y[(size_t)p * C + c] * f;
    }
    Z[(size_t)p * r + j] = sum;
}

// out = s * sum_m Y[m][c] Z[m][j]; layout 0: out[c][j] ([C][r]); 1: out[j][c] ([r][C]).
__global__ __launch_bounds__(256) void f32_grad(const float* __restrict__ Y, const float* __restrict__ Z,
                                               float* __restrict__ out, int M, int C, int r, float s,
                                               int layout, int accumulate) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)C * r) return;
    const int j = (int)(e / C), c = (int)(e % C);   // consecutive threads -> consecutive c
    float sum = 0.f;
    for (int m = 0; m < M; ++m) sum += Y[(size_t)m * C + c] * Z[(size_t)m * r + j];
    float v = s * sum;
    const size_t o = layout == 0 ? (size_t)c * r + j : (size_t)j * C + c;
    if (accumulate) v += out[o];
    out[o] = v;
}

}  // namespace lora
