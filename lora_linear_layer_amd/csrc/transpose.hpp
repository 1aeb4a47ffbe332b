// W^T of a frozen weight, made once so that the input-gradient GEMM reads its
// weight operand in the same [rows][contraction] layout as the forward GEMM
// (16-byte loads into the swizzled LDS tile, plain 16-byte fragment reads)
// instead of gathering it with transposing LDS reads.
#pragma once
#include "common.hpp"

namespace lora {

// Wt[k][n] = W[n][k] for W [N][K] bf16 (N, K multiples of 8): 64 x 64 tiles
// through LDS, 16-byte loads and stores.  Rows of the LDS tile are 144 bytes
// apart so that the column gathers of one store spread over the banks.
__global__ __launch_bounds__(256) void transpose_weight_kernel(const uint16_t* __restrict__ W,
                                                               uint16_t* __restrict__ Wt, int N, int K) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const int k0 = (int)blockIdx.x * 64, n0 = (int)blockIdx.y * 64;
    for (int u = threadIdx.x; u < 512; u += 256) {
        const int r = u >> 3, c = (u & 7) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + r < N && k0 + c < K) v = *reinterpret_cast<const u32x4*>(W + (size_t)(n0 + r) * K + k0 + c);
        *reinterpret_cast<u32x4*>(&tile[r][c]) = v;
    }
    __syncthreads();
    for (int u = threadIdx.x; u < 512; u += 256) {
        const int c = u >> 3, r = (u & 7) * 8;          // output row k0 + c, columns n0 + r .. n0 + r + 7
        if (k0 + c >= K || n0 + r >= N) continue;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (uint32_t)tile[r + 2 * i][c] | ((uint32_t)tile[r + 2 * i + 1][c] << 16);
        *reinterpret_cast<u32x4*>(Wt + (size_t)(k0 + c) * N + n0 + r) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

}  // namespace lora
