// Fused LoRA GEMM for gfx950: one kernel computes
//
//   Out[p][q] = sum_c L[p][c] * R(q, c)  +  s * sum_j E(q, j) * Z[p][j]
//   Z[p][j]   = sum_c L[p][c] * F(j, c)        (rank-r product, formed on chip)
//
// which is both directions of the LoRA linear layer:
//   forward  (page "ms-swift高效微调组合：LoRA+UnSloth提速实践", section 1.2
//            "算子融合": Linear, LoRA_A, LoRA_B and the add in one launch):
//            P=M, Q=N, C=K, L=X, R(q,c)=W[q][c], F(j,c)=A[j][c], E(q,j)=B[q][j], Z=U.
//   input gradient (page "Unsloth — 微调 2-5x 加速", section "核心要点", item 2:
//            (A B) dY evaluated as A (B dY)):
//            P=M, Q=K, C=N, L=dY, R(q,c)=W[c][q], F(j,c)=B[c][j], E(q,j)=A[j][q], Z=V.
// The 4-bit variants read R from codes + absmax + codebook and dequantise it
// while staging the tile (page "Unsloth — 微调 2-5x 加速", "核心要点" item 3).
//
// Tiling: a 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave
// owning 128 (q) x 128 (p) = 8 x 8 MFMA 16x16 tiles (256 fp32 accumulators per
// lane).  The contraction advances 64 at a time through double-buffered LDS
// stages (L tile 32 KB, R tile 32 KB, F tile RPAD*128 B); global loads for
// stage k+1 are in flight while stage k feeds the MFMAs.
// The rank-r product Z^T = F L^T reuses the L fragments already in registers
// (MFMA with F as the A operand), split between the two waves that share the
// same p rows.  In the epilogue the two halves meet in LDS and the update
// s * Z E^T is applied with MFMA: s*Z is split into bf16 hi + lo parts that sit
// in the two halves of the 32-long contraction, so the update keeps ~16
// mantissa bits of s*Z while E is exact in bf16.
// Edges: rows/columns outside P, Q and contraction chunks outside C are
// zero-filled on load and masked on store.  Requirements (checked on the
// host): C % 8 == 0 and Q % 8 == 0 (C % 64 == 0 and Q % 64 == 0 for 4-bit).
#pragma once
#include "common.hpp"

namespace lora {

enum FusedMode { kFwd = 0, kDx = 1, kQFwd = 2, kQDx = 3 };

struct FusedArgs {
    const uint16_t* L;      // [P][C] bf16
    const uint16_t* R;      // kFwd: [Q][C]; kDx: [C][Q] (bf16)
    const uint8_t* Rq;      // kQFwd: codes [Q][C/2]; kQDx: codes [C][Q/2]
    const uint16_t* Rabs;   // kQFwd: absmax [Q][C/64]; kQDx: absmax [C][Q/64] (fp16 bits)
    const float* codebook;  // [16]
    const uint16_t* F;      // kFwd/kQFwd: A [r][C]; kDx/kQDx: B [C][r]
    const uint16_t* E;      // kFwd/kQFwd: B [Q][r]; kDx/kQDx: A [r][Q]
    const float* Zin;       // precomputed Z [P][r] (ZIN variant), else unused
    uint16_t* Out;          // [P][Q] bf16
    float* Zsave;           // [P][r] float32 or nullptr
    int P, Q, C, r;
    float s;
};

constexpr int kBP = 256, kBQ = 256, kBK = 64, kThreads = 256;
constexpr int kTileBytes = kBP * kBK * 2;  // 32 KB per operand stage

template <int RPAD, bool ZIN>
struct FusedSmem {
    static constexpr int F_BYTES = ZIN ? 0 : RPAD * kBK * 2;
    static constexpr int STAGE = 2 * kTileBytes + F_BYTES;
    static constexpr int LUT = 256 * 8;  // byte -> (codebook[lo], codebook[hi]) for 4-bit modes
    static constexpr int TOTAL = 2 * STAGE + LUT;
    static_assert(256 * RPAD * 4 <= 2 * STAGE || ZIN, "Z exchange must fit in the stage buffers");
};

template <int MODE, int RPAD, bool ZIN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_lora_gemm(const FusedArgs a) {
    using SM = FusedSmem<RPAD, ZIN>;
    constexpr int JT = RPAD / 16;
    constexpr bool QUANT = (MODE == kQFwd || MODE == kQDx);
    constexpr bool TRANS = (MODE == kDx || MODE == kQDx);
    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wq = wave >> 1, wp = wave & 1;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int P = a.P, Q = a.Q, C = a.C, r = a.r;
    const int nPt = (P + kBP - 1) / kBP, nQt = (Q + kBQ - 1) / kBQ;
    int pt, qt;
    grouped_tile<4>(xcd_contiguous(blockIdx.x, nPt * nQt), nPt, nQt, pt, qt);
    const int p0 = pt * kBP, q0 = qt * kBQ;

    uint8_t* const lut = smem + 2 * SM::STAGE;
    if constexpr (QUANT) {
        const float lo = a.codebook[tid & 15], hi = a.codebook[tid >> 4];
        *reinterpret_cast<f32x2*>(lut + tid * 8) = f32x2{lo, hi};
        __syncthreads();
    }

    // ---------------------------------------------------------------- staging
    u32x4 regL[8];
    u32x4 regR[8];
    constexpr int F_CHUNKS = ZIN ? 0 : ((MODE == kFwd || MODE == kQFwd) ? (RPAD * 8 + kThreads - 1) / kThreads
                                                                        : RPAD / 4);
    uint32_t regF[F_CHUNKS > 0 ? (TRANS ? F_CHUNKS : 4 * F_CHUNKS) : 1];
    uint32_t regQ[QUANT ? 8 : 1];   // 4-bit: packed codes for this thread
    float regAbs[QUANT ? 8 : 1];

    auto load_stage = [&](int kt) {
        const int c0 = kt * kBK;
        // L tile: 256 rows x 8 chunks; chunk id = tid + 256 i
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = tid + kThreads * i;
            const int row = id >> 3, ch = id & 7;
            const int p = p0 + row, c = c0 + ch * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (p < P && c < C) v = *reinterpret_cast<const u32x4*>(a.L + (size_t)p * C + c);
            regL[i] = v;
        }
        if constexpr (MODE == kFwd) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int id = tid + kThreads * i;
                const int row = id >> 3, ch = id & 7;
                const int q = q0 + row, c = c0 + ch * 8;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (q < Q && c < C) v = *reinterpret_cast<const u32x4*>(a.R + (size_t)q * C + c);
                regR[i] = v;
            }
        } else if constexpr (MODE == kDx) {
            // W stored [C][Q]: 8 rows (c) x 8 columns (q) per thread, transposed on store
            const int qc = tid & 31, cg = tid >> 5;
            const int q = q0 + qc * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = c0 + cg * 8 + i;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (c < C && q < Q) v = *reinterpret_cast<const u32x4*>(a.R + (size_t)c * Q + q);
                regR[i] = v;
            }
        } else if constexpr (MODE == kQFwd) {
            // codes [Q][C/2]: thread tid owns row q0+tid, all 64 k of this stage (32 bytes)
            const int q = q0 + tid;
            if (q < Q) {
                const u32x4* src = reinterpret_cast<const u32x4*>(a.Rq + (size_t)q * (C >> 1) + (c0 >> 1));
                const u32x4 v0 = src[0], v1 = src[1];
                regQ[0] = v0[0]; regQ[1] = v0[1]; regQ[2] = v0[2]; regQ[3] = v0[3];
                regQ[4] = v1[0]; regQ[5] = v1[1]; regQ[6] = v1[2]; regQ[7] = v1[3];
                regAbs[0] = f16_bits_to_f32(a.Rabs[(size_t)q * (C >> 6) + (c0 >> 6)]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) regQ[i] = 0u;
                regAbs[0] = 0.f;
            }
        } else {  // kQDx: codes [C][Q/2]; 8 rows (c) x 8 q per thread
            const int qc = tid & 31, cg = tid >> 5;
            const int q = q0 + qc * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = c0 + cg * 8 + i;
                if (c < C && q < Q) {
                    regQ[i] = *reinterpret_cast<const uint32_t*>(a.Rq + (size_t)c * (Q >> 1) + (q >> 1));
                    regAbs[i] = f16_bits_to_f32(a.Rabs[(size_t)c * (Q >> 6) + (q >> 6)]);
                } else {
                    regQ[i] = 0u;
                    regAbs[i] = 0.f;
                }
            }
        }
        if constexpr (!ZIN) {
            if constexpr (MODE == kFwd || MODE == kQFwd) {
                // A [r][C]: RPAD rows x 8 chunks
#pragma unroll
                for (int i = 0; i < F_CHUNKS; ++i) {
                    const int id = tid + kThreads * i;
                    const int j = id >> 3, ch = id & 7;
                    const int c = c0 + ch * 8;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (j < r && c < C && id < RPAD * 8)
                        v = *reinterpret_cast<const u32x4*>(a.F + (size_t)j * C + c);
                    regF[4 * i + 0] = v[0]; regF[4 * i + 1] = v[1];
                    regF[4 * i + 2] = v[2]; regF[4 * i + 3] = v[3];
                }
            } else {
                // B [C][r] read transposed: element e = tid + 256 i -> (j = e / 64, c = e % 64)
#pragma unroll
                for (int i = 0; i < F_CHUNKS; ++i) {
                    const int e = tid + kThreads * i;
                    const int j = e >> 6, cl = e & 63;
                    const int c = c0 + cl;
                    regF[i] = (j < r && c < C) ? (uint32_t)a.F[(size_t)c * r + j] : 0u;
                }
            }
        }
    };

    // dequantise 8 packed codes (one dword, low nibble first) with one absmax
    auto decode8 = [&](uint32_t codes, float am) -> u32x4 {
        u32x4 out;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (codes >> (8 * b)) & 0xFFu;
            const f32x2 v = *reinterpret_cast<const f32x2*>(lut + byte * 8);
            out[b] = pack_bf16x2(v[0] * am, v[1] * am);
        }
        return out;
    };

    auto store_stage = [&](int stage) {
        uint8_t* const Ls = smem + stage * SM::STAGE;
        uint8_t* const Rs = Ls + kTileBytes;
        uint8_t* const Fs = Rs + kTileBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = tid + kThreads * i;
            *reinterpret_cast<u32x4*>(Ls + swz<128>(id >> 3, id & 7)) = regL[i];
        }
        if constexpr (MODE == kFwd) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int id = tid + kThreads * i;
                *reinterpret_cast<u32x4*>(Rs + swz<128>(id >> 3, id & 7)) = regR[i];
            }
        } else if constexpr (MODE == kDx) {
            u32x4 tr[8];
            transpose8x8_b16(regR, tr);
            const int qc = tid & 31, cg = tid >> 5;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<u32x4*>(Rs + swz<128>(qc * 8 + j, cg)) = tr[j];
        } else if constexpr (MODE == kQFwd) {
            const float am = regAbs[0];
#pragma unroll
            for (int ch = 0; ch < 8; ++ch)
                *reinterpret_cast<u32x4*>(Rs + swz<128>(tid, ch)) = decode8(regQ[ch], am);
        } else {
            u32x4 rows[8], tr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) rows[i] = decode8(regQ[i], regAbs[i]);
            transpose8x8_b16(rows, tr);
            const int qc = tid & 31, cg = tid >> 5;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<u32x4*>(Rs + swz<128>(qc * 8 + j, cg)) = tr[j];
        }
        if constexpr (!ZIN) {
            if constexpr (MODE == kFwd || MODE == kQFwd) {
#pragma unroll
                for (int i = 0; i < F_CHUNKS; ++i) {
                    const int id = tid + kThreads * i;
                    if (id < RPAD * 8) {
                        u32x4 v = {regF[4 * i], regF[4 * i + 1], regF[4 * i + 2], regF[4 * i + 3]};
                        *reinterpret_cast<u32x4*>(Fs + swz<128>(id >> 3, id & 7)) = v;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < F_CHUNKS; ++i) {
                    const int e = tid + kThreads * i;
                    const int j = e >> 6, cl = e & 63;
                    *reinterpret_cast<uint16_t*>(Fs + swz<128>(j, cl >> 3) + (cl & 7) * 2) = (uint16_t)regF[i];
                }
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 zacc[ZIN ? 1 : JT][4];
#pragma unroll
    for (int i = 0; i < (ZIN ? 1 : JT); ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) zacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (C + kBK - 1) / kBK;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_stage(kt + 1);
        const uint8_t* const Ls = smem + cur * SM::STAGE;
        const uint8_t* const Rs = Ls + kTileBytes;
        const uint8_t* const Fs = Rs + kTileBytes;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ch = kk * 4 + g4;
            bf16x8 rf[8], lf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                rf[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(Rs + swz<128>(wq * 128 + i * 16 + l16, ch)));
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lf[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(Ls + swz<128>(wp * 128 + i * 16 + l16, ch)));
#pragma unroll
            for (int qi = 0; qi < 8; ++qi)
#pragma unroll
                for (int pi = 0; pi < 8; ++pi) acc[qi][pi] = mfma16(rf[qi], lf[pi], acc[qi][pi]);
            if constexpr (!ZIN) {
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    const bf16x8 ff = as_bf16x8(*reinterpret_cast<const u32x4*>(Fs + swz<128>(jt * 16 + l16, ch)));
#pragma unroll
                    for (int pi = 0; pi < 4; ++pi) zacc[jt][pi] = mfma16(ff, lf[wq * 4 + pi], zacc[jt][pi]);
                }
            }
        }
        if (kt + 1 < nk) store_stage(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // Z exchange: Zx[p_local][j] float32, p_local in [0, 256), j in [0, RPAD)
    float* const Zx = reinterpret_cast<float*>(smem);
    if constexpr (!ZIN) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                const int pl = wp * 128 + (wq * 4 + pi) * 16 + l16;
                *reinterpret_cast<f32x4*>(Zx + pl * RPAD + jt * 16 + 4 * g4) = zacc[jt][pi];
            }
        __syncthreads();
        if (a.Zsave != nullptr && qt == 0) {
            for (int e = tid; e < kBP * r; e += kThreads) {
                const int pl = e / r, j = e - pl * r;
                if (p0 + pl < P) a.Zsave[(size_t)(p0 + pl) * r + j] = Zx[pl * RPAD + j];
            }
        }
    }

    const float s = a.s;
    constexpr int EJT = RPAD / 16;
#pragma unroll 1
    for (int jt = 0; jt < EJT; ++jt) {
        bf16x8 ef[8];
#pragma unroll
        for (int qi = 0; qi < 8; ++qi) {
            const int q = q0 + wq * 128 + qi * 16 + l16;
            uint32_t e4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + 4 * g4 + i;
                uint32_t v = 0u;
                if (q < Q && j < r) {
                    if constexpr (TRANS) v = a.E[(size_t)j * Q + q];
                    else v = a.E[(size_t)q * r + j];
                }
                e4[i] = v;
            }
            const u32x4 packed = {e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16),
                                  e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16)};
            ef[qi] = as_bf16x8(packed);
        }
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int pl = wp * 128 + pi * 16 + l16;
            f32x4 z;
            if constexpr (ZIN) {
                const int p = p0 + pl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = jt * 16 + 4 * g4 + i;
                    z[i] = (p < P && j < r) ? a.Zin[(size_t)p * r + j] : 0.f;
                }
            } else {
                z = *reinterpret_cast<const f32x4*>(Zx + pl * RPAD + jt * 16 + 4 * g4);
            }
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float zs = z[i] * s;
                const __bf16 h = (__bf16)zs;
                const float rem = zs - (float)h;
                hi[i] = __builtin_bit_cast(uint16_t, h);
                lo[i] = __builtin_bit_cast(uint16_t, (__bf16)rem);
            }
            const u32x4 zp = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                              lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
            const bf16x8 zf = as_bf16x8(zp);
#pragma unroll
            for (int qi = 0; qi < 8; ++qi) acc[qi][pi] = mfma16(ef[qi], zf, acc[qi][pi]);
        }
    }

    // store: lane holds Out[p][q .. q+3] for p = column, q = 4 consecutive rows
#pragma unroll
    for (int qi = 0; qi < 8; ++qi) {
        const int q = q0 + wq * 128 + qi * 16 + 4 * g4;
        if (q >= Q) continue;
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int p = p0 + wp * 128 + pi * 16 + l16;
            if (p < P) {
                const f32x4 v = acc[qi][pi];
                const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2*>(a.Out + (size_t)p * Q + q) = o;
            }
        }
    }
}

}  // namespace lora
