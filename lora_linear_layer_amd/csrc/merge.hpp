// Merge / unmerge of the adapter into the frozen weight (page "ms-swift框架下
// UnSloth与Liger-Kernel优化实战", section "设计权衡与最佳实践", item 4: before
// deployment the LoRA wrapper is removed and the adapter folded into W):
//   W_out[n][k] = W[n][k] + sgn * s * sum_j B[n][j] A[j][k]    (sgn = +1 merge, -1 unmerge)
// float32 arithmetic: the rank-r sum in increasing j (fused multiply-adds),
// times sgn * s, one add to W, then the tensor dtype (bf16: one RNE rounding).
//
// A workgroup (256 threads) owns a tile of 128 rows x 64 columns of W; thread
// t computes 8 consecutive columns (one 16-byte load and store in bf16) of the
// rows t / 8 + 32 i, i < 4, whose W values it requests first so that their
// latency overlaps the staging.  The tile's A columns [r][64] and B rows
// [128][r] are staged in LDS in the tensor dtype with 16-byte loads (B's rows
// are one contiguous block); each A row slice read from LDS serves four rows.
// HBM-bound at the pages' ranks: 2 + 2 bytes per bf16 weight, A and B small.
// W and W_out may be the same array: every element is read and written by one
// thread, the read first.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "lora_gemm.hpp"
#include "stream_store.hpp"

namespace lora {

constexpr int kMergeRows = 128, kMergeCols = 64, kMergeMaxR = 128, kMergeRpt = 4;

template <bool F32>
__global__ __launch_bounds__(256) void lora_merge_kernel(const void* W, const void* __restrict__ A,
                                                          const void* __restrict__ B, void* Wout, int N, int K,
                                                          int r, float scale) {
    using T = typename std::conditional<F32, float, uint16_t>::type;
    constexpr int EPC = 16 / sizeof(T);                   // elements per 16-byte chunk
    // As [j][c] (r x 64), Bs [i][j] (128 x r): sized by r in bf16 (dynamic LDS,
    // 384 r bytes, so that small ranks leave room for many workgroups per CU);
    // for the largest rank in the float32 checking mode
    T* As;
    T* Bs;
    if constexpr (F32) {
        __shared__ __attribute__((aligned(16))) float sA[kMergeMaxR * kMergeCols];
        __shared__ __attribute__((aligned(16))) float sB[kMergeRows * kMergeMaxR];
        As = sA;
        Bs = sB;
    } else {
        extern __shared__ __attribute__((aligned(16))) uint16_t merge_dyn[];
        As = merge_dyn;
        Bs = merge_dyn + r * kMergeCols;
    }
    const int tid = threadIdx.x;
    const int k0 = (int)blockIdx.x * kMergeCols, n0 = (int)blockIdx.y * kMergeRows;
    const int rg = tid >> 3, c8 = (tid & 7) * 8;
    const int k = k0 + c8;
    const T* const Wt = reinterpret_cast<const T*>(W);
    auto tof = [](T v) -> float {
        if constexpr (F32) return v;
        else return bf16_bits_to_f32(v);
    };
    // this thread's W values, kept as loaded (K % 8 == 0: the 8 columns are all
    // in range or all out)
    u32x4 w[kMergeRpt][F32 ? 2 : 1];
#pragma unroll
    for (int i = 0; i < kMergeRpt; ++i) {
        const int n = n0 + rg + 32 * i;
#pragma unroll
        for (int h = 0; h < (F32 ? 2 : 1); ++h) {
            w[i][h] = u32x4{0u, 0u, 0u, 0u};
            if (n < N && k < K) w[i][h] = *reinterpret_cast<const u32x4*>(Wt + (size_t)n * K + k + 4 * h);
        }
    }
    // A[j][k0 .. k0 + 63]: 64 / EPC chunks per rank row (columns past K read as zero)
    const T* const At = reinterpret_cast<const T*>(A);
    for (int c = tid; c < r * (kMergeCols / EPC); c += 256) {
        const int j = c / (kMergeCols / EPC), col = (c % (kMergeCols / EPC)) * EPC;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k0 + col < K) v = *reinterpret_cast<const u32x4*>(At + (size_t)j * K + k0 + col);   // K % 8 == 0
        *reinterpret_cast<u32x4*>(&As[j * kMergeCols + col]) = v;
    }
    // B rows n0 .. n0 + 127: one contiguous block of 128 r elements (16-byte aligned:
    // n0 r is a multiple of 128); rows past N read as zero
    const T* const Bt = reinterpret_cast<const T*>(B) + (size_t)n0 * r;
    const int valid = (min(N - n0, kMergeRows)) * r;
    for (int c = tid; c < kMergeRows * r / EPC; c += 256) {
        const int f = c * EPC;
        if (f + EPC <= valid) {
            *reinterpret_cast<u32x4*>(&Bs[f]) = *reinterpret_cast<const u32x4*>(Bt + f);
        } else {
            for (int e = 0; e < EPC; ++e) Bs[f + e] = f + e < valid ? Bt[f + e] : T(0);
        }
    }
    __syncthreads();
    float acc[kMergeRpt][8];
#pragma unroll
    for (int i = 0; i < kMergeRpt; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    for (int j = 0; j < r; ++j) {
        float a[8];
        if constexpr (F32) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(&As[j * kMergeCols + c8]);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(&As[j * kMergeCols + c8 + 4]);
            for (int e = 0; e < 4; ++e) { a[e] = a0[e]; a[4 + e] = a1[e]; }
        } else {
            const u32x4 v = *reinterpret_cast<const u32x4*>(&As[j * kMergeCols + c8]);
            for (int e = 0; e < 4; ++e) {
                a[2 * e] = bf16_bits_to_f32(v[e] & 0xFFFFu);
                a[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
            }
        }
#pragma unroll
        for (int i = 0; i < kMergeRpt; ++i) {
            const float b = tof(Bs[(rg + 32 * i) * r + j]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][e] = __builtin_fmaf(b, a[e], acc[i][e]);
        }
    }
#pragma unroll
    for (int i = 0; i < kMergeRpt; ++i) {
        const int n = n0 + rg + 32 * i;
        if (n >= N || k >= K) continue;
        float wv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (F32) {
                wv[e] = __uint_as_float(w[i][0][e]);
                wv[4 + e] = __uint_as_float(w[i][1][e]);
            } else {
                wv[2 * e] = bf16_bits_to_f32(w[i][0][e] & 0xFFFFu);
                wv[2 * e + 1] = bf16_bits_to_f32(w[i][0][e] >> 16);
            }
        }
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = wv[e] + scale * acc[i][e];
        if constexpr (F32) {
            float* const p = reinterpret_cast<float*>(Wout) + (size_t)n * K + k;
            store_stream(reinterpret_cast<f32x4*>(p), f32x4{out[0], out[1], out[2], out[3]});
            store_stream(reinterpret_cast<f32x4*>(p + 4), f32x4{out[4], out[5], out[6], out[7]});
        } else {
            store_stream(reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(Wout) + (size_t)n * K + k),
                         u32x4{pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]), pack_bf16x2(out[4], out[5]),
                               pack_bf16x2(out[6], out[7])});
        }
    }
}

// MFMA form of the bf16 merge for r >= 16, where the rank-r sum is a
// contraction worth the matrix cores and the form above is bound by its fused
// multiply-adds.  Same 128 x 64 tile and the same W loads and stores
// (thread t: 8 columns of rows t / 8 + 32 i).  Each wave forms 32 rows x 64
// columns of B A with v_mfma_f32_16x16x32_bf16: B's rows are read straight
// as fragments (8 consecutive j per lane), A's columns through
// ds_read_b64_tr_b16 from its [j][k] LDS rows, so a result lane holds 4
// consecutive columns of one row.  The float32 products meet in LDS (over the
// staged A and B) and are read back in the store layout.  RP = r rounded up
// to a multiple of 32; rank slots past r are zero.  float32 accumulation, one
// add to W, one rounding, as above; only the summation order of the rank-r
// sum differs.
template <int RP>
__global__ __launch_bounds__(256) void lora_merge_mfma(const uint16_t* W, const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B, uint16_t* Wout, int N,
                                                        int K, int r, float scale) {
    constexpr int ASTR = kMergeCols + 8;                  // A row stride in LDS (elements)
    constexpr int BSTR = RP + 8;                          // B row stride in LDS (elements)
    constexpr int CSTR = kMergeCols + 4;                  // float32 product row stride
    constexpr int AB_BYTES = (RP * ASTR + kMergeRows * BSTR) * 2, C_BYTES = kMergeRows * CSTR * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[AB_BYTES > C_BYTES ? AB_BYTES : C_BYTES];
    uint16_t* const As = reinterpret_cast<uint16_t*>(smem);
    uint16_t* const Bs = As + RP * ASTR;
    float* const Cs = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int k0 = (int)blockIdx.x * kMergeCols, n0 = (int)blockIdx.y * kMergeRows;
    const int rg = tid >> 3, c8 = (tid & 7) * 8, k = k0 + c8;
    u32x4 w[kMergeRpt];
#pragma unroll
    for (int i = 0; i < kMergeRpt; ++i) {
        const int n = n0 + rg + 32 * i;
        w[i] = u32x4{0u, 0u, 0u, 0u};
        if (n < N && k < K) w[i] = *reinterpret_cast<const u32x4*>(W + (size_t)n * K + k);
    }
    for (int c = tid; c < RP * (kMergeCols / 8); c += 256) {       // A[j][k0 .. k0 + 63]
        const int j = c / (kMergeCols / 8), col = (c % (kMergeCols / 8)) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < r && k0 + col < K) v = *reinterpret_cast<const u32x4*>(A + (size_t)j * K + k0 + col);
        *reinterpret_cast<u32x4*>(&As[j * ASTR + col]) = v;
    }
    for (int c = tid; c < kMergeRows * (RP / 8); c += 256) {       // B[n0 + i][j .. j + 7]
        const int i = c / (RP / 8), j = (c % (RP / 8)) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + i < N && j < r) {
            const uint16_t* const b = B + (size_t)(n0 + i) * r + j;
            if (r % 8 == 0) {                                  // 16-byte aligned rows
                v = *reinterpret_cast<const u32x4*>(b);
            } else {
                uint16_t e[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) e[t] = j + t < r ? b[t] : uint16_t(0);
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (uint32_t)e[2 * t] | ((uint32_t)e[2 * t + 1] << 16);
            }
        }
        *reinterpret_cast<u32x4*>(&Bs[i * BSTR + j]) = v;
    }
    __syncthreads();
    f32x4 acc[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[nb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js < RP / 32; ++js) {
        bf16x8 bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            bf[nb] = lds_b128(&Bs[(wave * 32 + nb * 16 + l16) * BSTR + js * 32 + 8 * g4]);
        // lane (l16, g4) gets A[js 32 + 8 g4 .. + 7][16 kb + l16]: its group's
        // 16 lanes address rank rows rlo .. rlo + 3, 4 columns each
        const int rlo = js * 32 + g4 * 8 + (l16 >> 2);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint16_t* const p = &As[rlo * ASTR + kb * 16 + (l16 & 3) * 4];
            const bf16x8 af = cat_tr(lds_tr4(p), lds_tr4(p + 4 * ASTR));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[nb][kb] = mfma16(af, bf[nb], acc[nb][kb]);
        }
    }
    __syncthreads();                                      // As, Bs no longer read: Cs overlays them
    // acc[nb][kb][v]: row 32 wave + 16 nb + l16, column 16 kb + 4 g4 + v
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            *reinterpret_cast<f32x4*>(&Cs[(wave * 32 + nb * 16 + l16) * CSTR + kb * 16 + 4 * g4]) = acc[nb][kb];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMergeRpt; ++i) {
        const int n = n0 + rg + 32 * i;
        if (n >= N || k >= K) continue;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(&Cs[(rg + 32 * i) * CSTR + c8]);
        const f32x4 p1 = *reinterpret_cast<const f32x4*>(&Cs[(rg + 32 * i) * CSTR + c8 + 4]);
        const float pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        float out[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = bf16_bits_to_f32(w[i][e] & 0xFFFFu) + scale * pr[2 * e];
            out[2 * e + 1] = bf16_bits_to_f32(w[i][e] >> 16) + scale * pr[2 * e + 1];
        }
        store_stream(reinterpret_cast<u32x4*>(Wout + (size_t)n * K + k),
                     u32x4{pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]), pack_bf16x2(out[4], out[5]),
                           pack_bf16x2(out[6], out[7])});
    }
}

}  // namespace lora
