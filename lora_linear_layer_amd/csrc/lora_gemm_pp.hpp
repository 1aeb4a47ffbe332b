// Fused LoRA GEMM for gfx950, ping-pong schedule: of the two waves that share
// each SIMD, one runs MFMAs while the other reads LDS and issues global loads,
// and they swap at every workgroup barrier.
//
// Same computation and operand roles as lora_gemm.hpp:
//   Out[p][q] = sum_c L[p][c] R(q, c)  +  s * sum_j E(q, j) Z[p][j]
//   Z[p][j]   = sum_c L[p][c] F(j, c)      (rank-r product, formed on chip)
// forward (page "ms-swift高效微调组合：LoRA+UnSloth提速实践", section 1.2
// "算子融合") with L=X, R=W, F=A, E=B, Z=U; input gradient (page "Unsloth —
// 微调 2-5x 加速", section "核心要点", item 2) with L=dY, R(q,c)=W[c][q],
// F(j,c)=B[c][j], E(q,j)=A[j][q], Z=V.
//
// Work split: a 256 (p) x 256 (q) tile per workgroup of 8 waves, 2 (p) x 4 (q),
// 128 p x 64 q per wave.  Waves 0-3 (group 0, p rows 0-127) and waves 4-7
// (group 1, p rows 128-255) put one wave on each SIMD.  The contraction
// advances 32 per step through a ring of 4 LDS slots (L 16 KB, R 16 KB,
// F RPAD x 64 B).  Per step a wave has a memory phase M (read its fragments
// of the step, issue its share of the loads of step + 3, wait for its share of
// step + 1) and a compute phase C (34 MFMAs).  Group 1 runs one phase behind
// group 0, so in every phase one wave of each SIMD feeds the MFMA pipe:
//     group 0:  M0 | C0 M1 | C1 M2 | ...
//     group 1:  -- | M0 C0 | M1 C1 | ...      ("|" = workgroup barrier)
// Group 0 stages the L tiles, group 1 the R and F tiles, each with
// buffer_load ... lds (global memory straight into LDS); a load of step t + 3
// has three memory phases of its issuer to land before anyone reads it.
//
// LDS layouts: contraction-contiguous tiles (L; R and F in forward) have rows
// of 32 values (64 B) with 16-byte chunk ch of row x at ch ^ ((x >> 1) & 3);
// in the input gradient R is W rows c (512 B) with 32-byte slots swizzled by
// sw512(c) and F is B rows c (RPAD values), both read with ds_read_b64_tr_b16.
#pragma once
#include "lora_gemm.hpp"

namespace lora {

namespace pp {
constexpr int BP = 256, BQ = 256, BK = 32, NT = 512, NSLOT = 4;
constexpr int TILE = BP * BK * 2;             // 16 KB per operand per step
}  // namespace pp

template <int RPAD, bool ZIN>
struct PPSmem {
    static constexpr int F_BYTES = ZIN ? 0 : RPAD * pp::BK * 2;
    static constexpr int SLOT = 2 * pp::TILE + F_BYTES;
    static constexpr int TOTAL = pp::NSLOT * SLOT;
    static_assert(F_BYTES == 0 || F_BYTES == 1024, "in-tile rank product needs RPAD == 16");
    static_assert(ZIN || pp::BP * RPAD * 4 <= TOTAL, "Z exchange must fit");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <bool TRANS, int RPAD, bool ZIN>
__global__ __launch_bounds__(pp::NT) void lora_gemm_pp(const GemmArgs a) {
    using namespace pp;
    using SM = PPSmem<RPAD, ZIN>;
    constexpr int JT = ZIN ? 1 : RPAD / 16;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SM::TOTAL];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave >> 2, gw = wave & 3;     // group, wave within the group
    const int wp = grp, wq = gw;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int P = a.P, Q = a.Q, C = a.C, r = a.r;
    const int nPt = (P + BP - 1) / BP, nQt = (Q + BQ - 1) / BQ;
    int pt, qt;
    grouped_tile<4>(xcd_contiguous(blockIdx.x, nPt * nQt), nPt, nQt, pt, qt);
    const int p0 = pt * BP, q0 = qt * BQ;

    // ------------------------------------------------------------ load plan
    // 64-byte row tiles: load i of a wave covers rows (4 gw + i) * 16 + lane / 4,
    // lane's chunk (lane % 4) ^ ((row >> 1) & 3) = (lane % 4) ^ ((lane >> 3) & 3).
    const int kc_row0 = gw * 64 + (lane >> 2);
    const int kc_ch = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;
    // group 0: L tile
    __amdgpu_buffer_rsrc_t rsT = make_rsrc(a.L + (size_t)p0 * C, (uint64_t)min(P - p0, BP) * C * 2);
    uint32_t offT = (uint32_t)(kc_row0 * C + kc_ch) * 2u;
    int chR0 = 0, chR1 = 0;
    if (grp == 1) {
        if constexpr (!TRANS) {
            rsT = make_rsrc(a.R + (size_t)q0 * C, (uint64_t)min(Q - q0, BQ) * C * 2);
        } else {
            // W rows c (512 bytes): load i covers rows (4 gw + i) * 2 + lane / 32
            const int pch = lane & 31;
            const int rowe = gw * 8 + (lane >> 5), rowo = rowe + 2;
            chR0 = (((pch >> 1) ^ sw512(rowe)) * 2 + (pch & 1)) * 8;
            chR1 = (((pch >> 1) ^ sw512(rowo)) * 2 + (pch & 1)) * 8;
            offT = (uint32_t)(rowe * Q) * 2u;
        }
    }
    // F tile (in-tile rank product): one 1 KB load, by wave 4
    const bool f_loader = !ZIN && wave == 4;
    __amdgpu_buffer_rsrc_t rsF = rsT;
    uint32_t offF = kOOB;
    int frow = 0, fch = 0;
    if constexpr (!ZIN) {
        if constexpr (!TRANS) {
            rsF = make_rsrc(a.F, (uint64_t)r * C * 2);
            frow = lane >> 2;                                          // j
            fch = kc_ch;
            offF = (uint32_t)(frow * C + fch) * 2u;
        } else {
            rsF = make_rsrc(a.F, (uint64_t)C * r * 2);
            frow = lane / (RPAD / 8);                                  // c within the step
            fch = (lane % (RPAD / 8)) * 8;                             // j
            offF = (uint32_t)(frow * r + fch) * 2u;
        }
    }
    const int lps = 4 + (f_loader ? 1 : 0);      // loads per step issued by this wave
    const int nk = (C + BK - 1) / BK;

    auto slot_of = [&](int t) { return smem + (t & (NSLOT - 1)) * SM::SLOT; };
    auto issue = [&](int t) {                     // this wave's share of step t's tiles
        const int c0 = t * BK;
        uint8_t* const Ls = slot_of(t);
        uint8_t* const dst = Ls + grp * TILE + gw * 4096;
        if (grp == 0 || !TRANS) {
            const bool ok = c0 + kc_ch < C;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                g2lds16(rsT, dst + i * 1024, ok ? offT + (uint32_t)(i * 16 * C + c0) * 2u : kOOB);
        } else {
            const int rows_left = min(C - c0, BK);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(a.R + (size_t)c0 * Q + q0, (uint64_t)(rows_left - 1) * Q * 2 + (uint64_t)(Q - q0) * 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = (i & 1) ? chR1 : chR0;
                g2lds16(rs, dst + i * 1024, (q0 + ch < Q) ? offT + (uint32_t)(2 * i * Q + ch) * 2u : kOOB);
            }
        }
        if constexpr (!ZIN) {
            if (f_loader) {
                uint32_t v;
                if constexpr (!TRANS) v = (frow < r && c0 + fch < C) ? offF + (uint32_t)c0 * 2u : kOOB;
                else v = (c0 + frow < C && fch < r) ? offF + (uint32_t)(c0 * r) * 2u : kOOB;
                g2lds16(rsF, Ls + 2 * TILE, v);
            }
        }
    };
    // wait until this wave's loads of step t have landed, given the steps issued after it
    auto wait_step = [&](int t) {
        const int younger = min(t + 2, nk - 1) - t;        // steps t+1 .. t+2 that exist
        if (younger >= 2) {
            if (lps == 5) vmcnt_le<10>(); else vmcnt_le<8>();
        } else if (younger == 1) {
            if (lps == 5) vmcnt_le<5>(); else vmcnt_le<4>();
        } else {
            vmcnt_le<0>();
        }
    };

    // ------------------------------------------------------------ fragments
    const int frag_off = l16 * 64 + ((g4 ^ ((l16 >> 1) & 3)) << 4);
    Frags<JT> fr;
    auto memory_phase = [&](int t) {
        const uint8_t* const Ls = slot_of(t);
        const uint8_t* const Rs = Ls + TILE;
        const uint8_t* const Fs = Rs + TILE;
#pragma unroll
        for (int i = 0; i < 8; ++i) fr.l[i] = lds_b128(Ls + (wp * 8 + ((i + 2 * wq) & 7)) * 1024 + frag_off);
        if constexpr (!TRANS) {
#pragma unroll
            for (int i = 0; i < 4; ++i) fr.r[i] = lds_b128(Rs + (wq * 4 + i) * 1024 + frag_off);
        } else {
            const int rlo = g4 * 8 + (l16 >> 2);
            const uint8_t* const base = Rs + rlo * 512 + (l16 & 3) * 8;
            const int sw = sw512(rlo);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint8_t* const p = base + (((wq * 4 + i) ^ sw) << 5);
                fr.r[i] = cat_tr(lds_tr4(p), lds_tr4(p + 4 * 512));
            }
        }
        if constexpr (!ZIN) {
            if constexpr (!TRANS) {
                fr.f[0] = lds_b128(Fs + frag_off);
            } else {
                const int rlo = g4 * 8 + (l16 >> 2);
                const uint8_t* const p = Fs + rlo * (RPAD * 2) + (l16 & 3) * 8;
                fr.f[0] = cat_tr(lds_tr4(p), lds_tr4(p + 4 * RPAD * 2));
            }
        }
        if (t + 3 < nk) issue(t + 3);
        if (t + 1 < nk) wait_step(t + 1);
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 zacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    auto compute_phase = [&]() {
#pragma unroll
        for (int pi = 0; pi < 8; ++pi)
#pragma unroll
            for (int qi = 0; qi < 4; ++qi) acc[qi][pi] = mfma16(fr.r[qi], fr.l[pi], acc[qi][pi]);
        if constexpr (!ZIN) {
#pragma unroll
            for (int z = 0; z < 2; ++z) zacc[z] = mfma16(fr.f[0], fr.l[z], zacc[z]);
        }
    };

    // ------------------------------------------------------------ main loop
#pragma unroll
    for (int t = 0; t < 3; ++t)
        if (t < nk) issue(t);
    wait_step(0);
    lds_barrier();
    if (grp == 0) memory_phase(0);
    lds_barrier();
    if (grp == 0) {
        for (int t = 0; t < nk; ++t) {
            compute_phase();
            lds_barrier();
            if (t + 1 < nk) memory_phase(t + 1);
            lds_barrier();
        }
    } else {
        for (int t = 0; t < nk; ++t) {
            memory_phase(t);
            lds_barrier();
            compute_phase();
            lds_barrier();
        }
    }

    // ------------------------------------------------------------ epilogue
    float* const Zx = reinterpret_cast<float*>(smem);   // [256][RPAD] float32
    if constexpr (!ZIN) {
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            const int pl = wp * 128 + (wq * 2 + z) * 16 + l16;
            *reinterpret_cast<f32x4*>(Zx + pl * RPAD + 4 * g4) = zacc[z];
        }
        lds_barrier();
        if (a.Zsave != nullptr && qt == 0) {
            for (int e = tid; e < BP * r; e += NT) {
                const int pl = e / r, j = e - pl * r;
                if (p0 + pl < P) a.Zsave[(size_t)(p0 + pl) * r + j] = Zx[pl * RPAD + j];
            }
        }
    }

    const float s = a.s;
#pragma unroll 1
    for (int jt = 0; jt < RPAD / 16; ++jt) {
        bf16x8 ef[4];
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) {
            const int q = q0 + wq * 64 + qi * 16 + l16;
            uint32_t e4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + 4 * g4 + i;
                uint32_t v = 0u;
                if (q < Q && j < r) v = TRANS ? a.E[(size_t)j * Q + q] : a.E[(size_t)q * r + j];
                e4[i] = v;
            }
            const uint32_t w0 = e4[0] | (e4[1] << 16), w1 = e4[2] | (e4[3] << 16);
            ef[qi] = as_bf16x8(u32x4{w0, w1, w0, w1});
        }
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int pl = wp * 128 + ((pi + 2 * wq) & 7) * 16 + l16;
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
                hi[i] = __builtin_bit_cast(uint16_t, h);
                lo[i] = __builtin_bit_cast(uint16_t, (__bf16)(zs - (float)h));
            }
            const bf16x8 zf = as_bf16x8(u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                              lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)});
#pragma unroll
            for (int qi = 0; qi < 4; ++qi) acc[qi][pi] = mfma16(ef[qi], zf, acc[qi][pi]);
        }
    }

#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
        const int q = q0 + wq * 64 + qi * 16 + 4 * g4;
        if (q >= Q) continue;
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int p = p0 + wp * 128 + ((pi + 2 * wq) & 7) * 16 + l16;
            if (p < P) {
                const f32x4 v = acc[qi][pi];
                const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2*>(a.Out + (size_t)p * Q + q) = o;
            }
        }
    }
}

}  // namespace lora
