// Adapter gradients as split-M reductions over tokens (page "ms-swift高效微调组合：
// LoRA+UnSloth提速实践", section 1.2 "梯度计算绕过Autograd": closed-form LoRA
// gradients; the printed formulas omit the input and the scale, the forms
// here are the exact ones):
//
//   G[c][j] = sum_m Y[m][c] * Z[m][j]
//   dA[j][k] = s * G  with Y = X  [M][K], Z = V = dY B   (output [r][K])
//   dB[n][j] = s * G  with Y = dY [M][N], Z = U = X A^T  (output [N][r])
//
// Stage 1 (grad_partials): workgroup (c block of 128, m block) streams its Y
// rows once from HBM, transposes 8x8 sub-blocks in registers so the token
// index becomes the MFMA contraction, and accumulates G with MFMA (Z split into
// bf16 hi + lo, Y exact in bf16).  Each m block writes its own float32
// partial; no atomics.
// Stage 2 (grad_reduce): one thread per output element sums the partials in
// increasing m-block order, scales by s and writes the output dtype.  The
// result is bitwise reproducible from run to run.
#pragma once
#include "common.hpp"

namespace lora {

struct GradProblem {
    const uint16_t* Y;  // [M][C] bf16
    const float* Z;     // [M][r] float32
    float* part;        // [n_mblk][C][r] float32
    int C;
    int n_cblk;         // ceil(C / 128)
};

struct GradArgs {
    GradProblem prob[2];
    int n_prob;
    int M, r;
    int mblk_rows;      // multiple of 128
    int n_mblk;
};

constexpr int kGradCB = 128, kGradMB = 128;

template <int RPAD>
__global__ __launch_bounds__(256) void grad_partials(const GradArgs a) {
    constexpr int JT = RPAD / 16;
    // Yt[c][m]: 128 rows x 256 B; Zh/Zl[j][m]: RPAD rows x 256 B
    __shared__ __attribute__((aligned(16))) uint8_t smem[kGradCB * 256 + 2 * RPAD * 256];
    uint8_t* const Yt = smem;
    uint8_t* const Zh = smem + kGradCB * 256;
    uint8_t* const Zl = Zh + RPAD * 256;

    const int pidx = blockIdx.z;
    if (pidx >= a.n_prob) return;
    const GradProblem pr = a.prob[pidx];
    if ((int)blockIdx.x >= pr.n_cblk) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int M = a.M, C = pr.C, r = a.r;
    const int c0 = blockIdx.x * kGradCB;
    const int m_begin = blockIdx.y * a.mblk_rows;
    const int m_end = min(M, m_begin + a.mblk_rows);

    f32x4 acc[2][JT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // per-thread Y sub-block: 8 rows (m) x 8 columns (c)
    const int cc = tid & 15, mg = tid >> 4;
    constexpr int ZE = RPAD * kGradMB / 256;  // Z elements per thread per step
    u32x4 ry[8];
    float rz[ZE];

    auto load = [&](int m0) {
        const int c = c0 + cc * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = m0 + mg * 8 + i;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (m < m_end && c < C) v = *reinterpret_cast<const u32x4*>(pr.Y + (size_t)m * C + c);
            ry[i] = v;
        }
#pragma unroll
        for (int i = 0; i < ZE; ++i) {
            const int e = tid + 256 * i;
            const int ml = e / RPAD, j = e % RPAD;
            const int m = m0 + ml;
            rz[i] = (m < m_end && j < r) ? pr.Z[(size_t)m * r + j] : 0.f;
        }
    };
    auto store = [&]() {
        u32x4 tr[8];
        transpose8x8_b16(ry, tr);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<u32x4*>(Yt + swz<256>(cc * 8 + j, mg)) = tr[j];
#pragma unroll
        for (int i = 0; i < ZE; ++i) {
            const int e = tid + 256 * i;
            const int ml = e / RPAD, j = e % RPAD;
            const float z = rz[i];
            const __bf16 h = (__bf16)z;
            const __bf16 l = (__bf16)(z - (float)h);
            const uint32_t off = swz<256>(j, ml >> 3) + (ml & 7) * 2;
            *reinterpret_cast<__bf16*>(Zh + off) = h;
            *reinterpret_cast<__bf16*>(Zl + off) = l;
        }
    };

    if (m_begin < m_end) load(m_begin);
    for (int m0 = m_begin; m0 < m_end; m0 += kGradMB) {
        store();
        __syncthreads();
        if (m0 + kGradMB < m_end) load(m0 + kGradMB);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int ch = kk * 4 + g4;
            bf16x8 yf[2];
#pragma unroll
            for (int ci = 0; ci < 2; ++ci)
                yf[ci] = as_bf16x8(*reinterpret_cast<const u32x4*>(Yt + swz<256>(wave * 32 + ci * 16 + l16, ch)));
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const bf16x8 zh = as_bf16x8(*reinterpret_cast<const u32x4*>(Zh + swz<256>(jt * 16 + l16, ch)));
                const bf16x8 zl = as_bf16x8(*reinterpret_cast<const u32x4*>(Zl + swz<256>(jt * 16 + l16, ch)));
#pragma unroll
                for (int ci = 0; ci < 2; ++ci) {
                    acc[ci][jt] = mfma16(yf[ci], zh, acc[ci][jt]);
                    acc[ci][jt] = mfma16(yf[ci], zl, acc[ci][jt]);
                }
            }
        }
        __syncthreads();
    }

    // lane holds G[c = base + 4 g + i][j = jt*16 + l16]
    float* const out = pr.part + (size_t)blockIdx.y * C * r;
#pragma unroll
    for (int ci = 0; ci < 2; ++ci)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const int j = jt * 16 + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + wave * 32 + ci * 16 + 4 * g4 + i;
                if (c < C && j < r) out[(size_t)c * r + j] = acc[ci][jt][i];
            }
        }
}

struct ReduceProblem {
    const float* part;  // [n_mblk][C][r]
    void* out;          // layout 0: [C][r]; layout 1: [r][C]
    int C;
    int layout;
};

struct ReduceArgs {
    ReduceProblem prob[2];
    int n_prob;
    int r, n_mblk;
    float s;
    int f32_out;    // 0: bf16, 1: float32
    int accumulate; // add into the existing output
};

__global__ __launch_bounds__(256) void grad_reduce(const ReduceArgs a) {
    const int pidx = blockIdx.y;
    if (pidx >= a.n_prob) return;
    const ReduceProblem pr = a.prob[pidx];
    const int r = a.r;
    const size_t total = (size_t)pr.C * r;
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    float sum = 0.f;
    for (int b = 0; b < a.n_mblk; ++b) sum += pr.part[(size_t)b * total + e];
    float v = sum * a.s;
    const int c = (int)(e / r), j = (int)(e % r);
    const size_t o = pr.layout == 0 ? e : (size_t)j * pr.C + c;
    if (a.f32_out) {
        float* out = reinterpret_cast<float*>(pr.out);
        if (a.accumulate) v += out[o];
        out[o] = v;
    } else {
        uint16_t* out = reinterpret_cast<uint16_t*>(pr.out);
        if (a.accumulate) v += bf16_bits_to_f32(out[o]);
        const __bf16 h = (__bf16)v;
        out[o] = __builtin_bit_cast(uint16_t, h);
    }
}

// Skinny rank-r product Z[p][j] = sum_c Y[p][c] * F(j, c) with float32 output,
// used when U = X A^T or V = dY B is needed outside the fused GEMM (large r,
// no saved U, no dX).  F_TRANS = false: F = A [r][C]; F_TRANS = true:
// F(j, c) = B[c][j] with B [C][r].  HBM-bound on Y.
// Workgroup (x, y) of 4 waves owns 64 rows and the contraction chunk
// [y * chunk, (y + 1) * chunk); it writes its partial sums to
// Z + y * P * r (gridDim.y == 1: the result itself), and skinny_sum adds the
// chunks in a fixed order.
template <int RPAD, bool F_TRANS>
__global__ __launch_bounds__(256) void skinny_rank(const uint16_t* __restrict__ Y, const uint16_t* __restrict__ F,
                                                  float* __restrict__ Zall, int P, int C, int r, int chunk) {
    float* const Z = Zall + (size_t)blockIdx.y * P * r;
    const int c_begin = blockIdx.y * chunk, c_end = min(C, c_begin + chunk);
    constexpr int JT = RPAD / 16;
    __shared__ __attribute__((aligned(16))) uint8_t smem[64 * 128 + RPAD * 128];
    uint8_t* const Ys = smem;
    uint8_t* const Fs = smem + 64 * 128;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int p0 = blockIdx.x * 64;
    f32x4 acc[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = c_begin; c0 < c_end; c0 += 64) {
        // Y tile 64 x 64: 512 chunks, 2 per thread
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int id = tid + 256 * i;
            const int row = id >> 3, ch = id & 7;
            const int p = p0 + row, c = c0 + ch * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (p < P && c < c_end) v = *reinterpret_cast<const u32x4*>(Y + (size_t)p * C + c);
            *reinterpret_cast<u32x4*>(Ys + swz<128>(row, ch)) = v;
        }
        if constexpr (!F_TRANS) {
            for (int id = tid; id < RPAD * 8; id += 256) {
                const int j = id >> 3, ch = id & 7;
                const int c = c0 + ch * 8;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (j < r && c < c_end) v = *reinterpret_cast<const u32x4*>(F + (size_t)j * C + c);
                *reinterpret_cast<u32x4*>(Fs + swz<128>(j, ch)) = v;
            }
        } else {
            for (int e = tid; e < RPAD * 64; e += 256) {
                const int j = e >> 6, cl = e & 63;
                const int c = c0 + cl;
                const uint16_t v = (j < r && c < c_end) ? F[(size_t)c * r + j] : (uint16_t)0;
                *reinterpret_cast<uint16_t*>(Fs + swz<128>(j, cl >> 3) + (cl & 7) * 2) = v;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ch = kk * 4 + g4;
            const bf16x8 yf = as_bf16x8(*reinterpret_cast<const u32x4*>(Ys + swz<128>(wave * 16 + l16, ch)));
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const bf16x8 ff = as_bf16x8(*reinterpret_cast<const u32x4*>(Fs + swz<128>(jt * 16 + l16, ch)));
                acc[jt] = mfma16(ff, yf, acc[jt]);
            }
        }
        __syncthreads();
    }
    // lane holds Z^T[j = jt*16 + 4 g + i][p = p0 + wave*16 + l16]
    const int p = p0 + wave * 16 + l16;
    if (p < P) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + 4 * g4 + i;
                if (j < r) Z[(size_t)p * r + j] = acc[jt][i];
            }
    }
}

// Z[e] = sum over the n_parts partials of skinny_rank, in increasing chunk order.
__global__ __launch_bounds__(256) void skinny_sum(const float* __restrict__ part, float* __restrict__ Z, int64_t n,
                                                 int n_parts) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    float sum = 0.f;
    for (int k = 0; k < n_parts; ++k) sum += part[(size_t)k * n + e];
    Z[e] = sum;
}

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
