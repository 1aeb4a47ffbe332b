// Rank-r products that stream a large bf16 matrix Y [M][C] from HBM once:
//
//   rank_stream:    G[c][j] = sum_m Y[m][c] Z2[m][j]   (dA^T = X^T V / s, dB = dY^T U / s)
//   rank_z_lds:     Z[m][j] = sum_c Y[m][c] F(j, c)    (U = X A^T, V = dY B)
//
// These are the adapter-gradient products of the backward (page "ms-swift高效微调
// 组合：LoRA+UnSloth提速实践", section 1.2 "梯度计算绕过Autograd": closed-form
// LoRA gradients; the printed formulas omit the input and the scale, the
// forms here are the exact vector-Jacobian products) and the stand-alone
// rank-r products U and V (page "Unsloth — 微调 2-5x 加速", section "核心要点",
// item 2: only [M, r] intermediates are formed).
//
// Both are HBM-bound.  A rank_stream workgroup (4 waves) owns one 128-wide
// tile of c and a chunk of the tokens m, walks the chunk in steps of TM x 128 of
// Y (TM = 128 tokens for r <= 16, else 64) that arrive through a
// double-buffered LDS ring straight from global memory
// (buffer_load ... lds, rows of 256 bytes, 16-byte chunk ch of row x at
// ch ^ y_swz(x)), and writes a float32 partial per chunk; grad_final adds the
// chunks in a fixed order, so results are bitwise reproducible.  MFMA
// 16x16x32 bf16 with float32 accumulation; Y^T fragments are gathered with
// ds_read_b64_tr_b16.  The rank-side operand arrives the same way, as the two
// bf16 planes hi = bf16(Z2^T), lo = bf16(Z2^T - hi) of [r][Mp] (tokens padded
// with zeros to a multiple of 128, stored token-block major as zt_index gives),
// which zt_hilo writes from Z2 [M][r] float32.
#pragma once
#include "lora_gemm.hpp"

namespace lora {

constexpr int kRT = 128;      // tile edge (rows of Y x columns of Y)

// One product G[c][j] = sum_m Y[m][c] Z2[m][s_j0 + j], c < C, j < rl (at most RPAD),
// into part[chunk * chunk_stride + c * out_r + out_j0 + j].
struct RankProblem {
    const uint16_t* Y;      // [M][C] bf16, row stride ldy
    const uint16_t* S;      // hi plane of Z2^T, bf16 [s_rows][Mp] in zt_index order
    const uint16_t* S_lo;   // lo plane of Z2^T (same shape)
    float* part;            // token-chunk partials, chunk_stride floats apart
    int C, ldy;
    int n_tiles;            // 128-wide tiles of c
    int s_rows, s_j0;       // rows of the planes, first plane row used
    int rl;                 // rank columns of this problem
    int out_r, out_j0;
    size_t chunk_stride;
};

constexpr int kMaxRankProblems = 8;

struct RankArgs {
    RankProblem prob[kMaxRankProblems];
    int n_prob;
    int M;
    int chunk_tiles;        // contraction tiles per chunk
    int n_chunk;
};

// A ring step covers TM tokens: 128 for r <= 16, 64 above, where the
// Z2 hi / lo tiles grow with the rank and 128-token stages would leave one
// workgroup (one stage in flight) per CU; with 64-token steps two or three fit.
template <int RPAD>
struct RankSmem {
    static constexpr int TM = RPAD <= 16 ? kRT : kRT / 2;
    static constexpr int YT = TM * kRT * 2;           // Y tile: TM rows of 256 bytes
    static constexpr int SIDE = RPAD * TM * 2;        // one of the Z2 hi / lo tiles: RPAD rows of 2 TM bytes
    static constexpr int STAGE = YT + 2 * SIDE;
    static constexpr int TOTAL = 2 * STAGE;
    static_assert(RPAD <= 64 && TOTAL <= 80 * 1024, "LDS budget: two workgroups per CU");
};

// LDS chunk swizzles (16-byte chunk ch of a row stored at ch ^ swz(row)),
// chosen so that the fragment reads hit distinct banks:
//  - Y rows (256 bytes): one transposing read's 32 lanes of a bank window read
//    rows m0 + y and m0 + 8 + y (y < 4), two chunks of each; row bits 0-1 and 3
//    spread them over all 16 chunks.  (row & 7 left rows 8 apart on the same
//    chunks: 4-way conflicts.)
//  - side rows of 2 TM bytes: one 16-byte read's 16 lanes read rows j .. j + 15
//    at one chunk; 256-byte rows use j & 15, 128-byte rows (two per bank window)
//    (j >> 1) & 7.  (j & 7 paired rows 8 apart: 2-way.)
__device__ __forceinline__ int y_swz(int row) { return ((row & 3) << 1) | (((row >> 3) & 1) << 3); }
template <int TM>
__device__ __forceinline__ int side_swz(int row) {
    static_assert(TM == 128 || TM == 64, "side rows of 256 or 128 bytes");
    if constexpr (TM == 128) return row & 15;
    else return (row >> 1) & 7;
}

// Problem blockIdx.z, output tile blockIdx.x, token chunk blockIdx.y.
template <int RPAD>
__global__ __launch_bounds__(256) void rank_stream(const RankArgs a) {
    using SM = RankSmem<RPAD>;
    constexpr int JT = RPAD / 16;
    constexpr int TM = SM::TM;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SM::TOTAL];

    const int pidx = blockIdx.z;
    if (pidx >= a.n_prob) return;
    const RankProblem pr = a.prob[pidx];
    if ((int)blockIdx.x >= pr.n_tiles) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int M = a.M, C = pr.C, ldy = pr.ldy;
    const int rl = min(pr.rl, RPAD);                   // rank columns of this problem
    // the output tile c0 = o0; token tiles [t_begin, t_end) of 128, walked in
    // steps of TM tokens: [s_begin, s_end)
    const int o0 = blockIdx.x * kRT;
    const int n_ct = (M + kRT - 1) / kRT;
    const int t_begin = blockIdx.y * a.chunk_tiles;
    const int t_end = min(n_ct, t_begin + a.chunk_tiles);
    const int s_begin = t_begin * (kRT / TM);
    const int s_end = min((M + TM - 1) / TM, t_end * (kRT / TM));

    // Y tile of step t: TM rows m, columns c (256 bytes per row); wave w issues
    // loads b = TM/16 w .. + TM/16 - 1, each 4 rows: row = 4 b + lane / 16
    constexpr int YLW = TM / 16;                      // Y loads per wave
    auto issue_y = [&](int t, uint8_t* Ys) {
        const int m0 = t * TM;
        const int c0 = o0;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(pr.Y + (size_t)m0 * ldy + c0, stream_y_bytes(M, C, m0, c0, TM, ldy));
#pragma unroll
        for (int i = 0; i < YLW; ++i) {
            const int b = wave * YLW + i;
            const int row = 4 * b + (lane >> 4);
            const int ch = ((lane & 15) ^ y_swz(row)) * 8;
            g2lds16<true>(rs, Ys + b * 1024, (c0 + ch < C) ? (uint32_t)(row * ldy + ch) * 2u : kOOB);
        }
    };
    // side tile(s) of step t: plane rows s_j0 .. s_j0 + RPAD - 1 of S (and S_lo), tokens
    // t TM .. + TM - 1, which lie in one 128-token block of the planes (rows
    // 256 bytes apart there); in LDS rows of 2 TM bytes whose 16-byte chunk ch of
    // row x sits at ch ^ side_swz(x).  The resources start at row s_j0 of the
    // step's block, so their range is a few KB whatever M is.  Wave w issues
    // loads b = SLW w .. of each plane, each SRL rows: row = SRL b + lane / (TM / 8)
    constexpr int SLW = RPAD * TM / 2048;             // side loads per wave per plane
    constexpr int SRL = 1024 / (2 * TM);              // side rows per 1 KB load
    static_assert(SLW >= 1, "side tile smaller than one load per wave");
    static_assert(kSideBlock % TM == 0, "a step stays inside one token block");
    const uint64_t side_range = stream_side_bytes(rl, TM);
    auto issue_side = [&](int t, uint8_t* Ss) {
        const int64_t m0 = (int64_t)t * TM;
        const size_t base = zt_index(pr.s_j0, m0, pr.s_rows);
        const __amdgpu_buffer_rsrc_t rsS = make_rsrc(pr.S + base, side_range);
        const __amdgpu_buffer_rsrc_t rsSl = make_rsrc(pr.S_lo + base, side_range);
#pragma unroll
        for (int i = 0; i < SLW; ++i) {
            const int b = wave * SLW + i;
            const int row = SRL * b + lane / (TM / 8);
            const int ch = ((lane % (TM / 8)) ^ side_swz<TM>(row)) * 8;
            const uint32_t off = row < rl ? (uint32_t)(row * kSideBlock + ch) * 2u : kOOB;
            g2lds16<true>(rsS, Ss + b * 1024, off);
            g2lds16<true>(rsSl, Ss + SM::SIDE + b * 1024, off);
        }
    };

    f32x4 acc[JT][2];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt][0] = acc[jt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: step s_begin in slot 0
    if (s_begin < s_end) {
        issue_y(s_begin, smem);
        issue_side(s_begin, smem + SM::YT);
    }
    vmcnt_le<0>();
    __syncthreads();
    for (int t = s_begin; t < s_end; ++t) {
        uint8_t* const cur = smem + ((t - s_begin) & 1) * SM::STAGE;
        uint8_t* const nxt = smem + ((t - s_begin + 1) & 1) * SM::STAGE;
        const bool more = t + 1 < s_end;
        if (more) {
            issue_y(t + 1, nxt);
            issue_side(t + 1, nxt + SM::YT);
        }
        const uint8_t* const Ys = cur;
        const uint8_t* const Ss = cur + SM::YT;
        // wave w owns output blocks 2w and 2w + 1 (16 rows each) of the 128-wide tile
#pragma unroll
        for (int kk = 0; kk < TM / 32; ++kk) {
            // B operand: Y^T, columns c = l16 of block, 8 consecutive m from rows kk*32 + 8 g4 ..
            bf16x8 yf[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
                const int c = (2 * wave + z) * 16 + (l16 & 3) * 4;
                const int mlo = kk * 32 + g4 * 8 + (l16 >> 2);
                const int mhi = mlo + 4;
                const i16x4 lo = lds_tr4(Ys + mlo * 256 + (((c >> 3) ^ y_swz(mlo)) << 4) + (c & 7) * 2);
                const i16x4 hi = lds_tr4(Ys + mhi * 256 + (((c >> 3) ^ y_swz(mhi)) << 4) + (c & 7) * 2);
                yf[z] = cat_tr(lo, hi);
            }
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const int j = jt * 16 + l16;
                const int off = j * (2 * TM) + (((kk * 4 + g4) ^ side_swz<TM>(j)) << 4);
                const bf16x8 sa = lds_b128(Ss + off);
                const bf16x8 sl = lds_b128(Ss + SM::SIDE + off);
#pragma unroll
                for (int z = 0; z < 2; ++z) acc[jt][z] = mfma16(sa, yf[z], acc[jt][z]);
#pragma unroll
                for (int z = 0; z < 2; ++z) acc[jt][z] = mfma16(sl, yf[z], acc[jt][z]);
            }
        }
        vmcnt_le<0>();
        __syncthreads();
    }

    // lane holds out^T rows j = jt*16 + 4 g4 + i at column o = block*16 + l16
    const int olim = C;
    float* const out = pr.part + (size_t)blockIdx.y * pr.chunk_stride;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            const int o = o0 + (2 * wave + z) * 16 + l16;
            if (o >= olim) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + 4 * g4 + i;
                if (j < rl) out[(size_t)o * pr.out_r + pr.out_j0 + j] = acc[jt][z][i];
            }
        }
}

// Z with the rank side in LDS: Z[m][z_j0 + j] = sum_c Y[m][c] F[f_j0 + j][c] for
// j < rl (F bf16 rows [f_rows][C], row stride C; Y [M][C] with row stride ldy).
// Workgroup (x, y): 8 waves; wave w owns rows m = 128 x + 16 w + (0 .. 15) (one MFMA
// row block) and the workgroup the contraction chunk y, [cb, ce), chunk_c columns (a
// multiple of SC).  Y is addressed from the workgroup's first row (a 128-row
// block stays below 2^29 bytes), so Y itself may exceed 2 GB.  F comes in
// SC-column slices (16 JB rows each) through a double-buffered LDS pair (row j
// of a slice: 2 SC bytes, 16-byte chunk ch stored at ch ^ (j % 16), so the 16
// rows one fragment read touches hit distinct banks); each lane loads its Y
// fragment (8 consecutive c of one row, 16 bytes) straight from global memory
// into registers, D = SC / 32 steps of 32 columns ahead.  Every Y fragment
// feeds JB MFMAs, so one pass over Y forms up to 16 JB rank columns (JB = 12:
// 192, with 128-column slices to stay within LDS).  Out-of-range rows, columns
// and rank rows read zero.  Writes out[y * chunk_stride + m * z_ld + z_j0 + j].
// The linears of a group run as one launch, member blockIdx.z: each with its
// own columns of Y (the member's columns of dY), its F, its contraction chunks
// and its output (its rank columns of Z, or its own region of partials).
struct RankZMember {
    const uint16_t* Y;        // the member's first column of Y
    const uint16_t* F;
    float* out;
    const float* row_scale;   // optional scale of each output row (when out is Z itself)
    size_t chunk_stride;      // floats between the partials of two contraction chunks
    int C, z_ld, z_j0, chunk_c, n_used;
};

struct RankZArgs {
    RankZMember mem[kMaxMembers];
    int ldy, M, f_j0, rl;
    int f_ld;                 // FB: row stride of F given as B [C][f_ld] (rank columns contiguous)
};

// FB = true: F(j, c) = B[c][f_j0 + j] from B's own rows (f_ld = its row stride,
// a multiple of 8), so that V = dY B needs no transposed copy of B: the slice
// holds SC rows c of 32 JB bytes (rank columns 0 .. 16 JB - 1, zeros past rl),
// and the fragments are gathered down its columns with ds_read_b64_tr_b16, as
// the input-gradient GEMM gathers B.  One such read touches rows c, c + 1, c + 2,
// c + 3 and the same four 8 rows on, 32 bytes each; to give those 8 rows 8
// distinct bank groups, the 32-byte column slot s of row c is stored at
// s ^ fb_swz(c) (JB >= 2), and with one slot per row (JB = 1) row c at
// fb_row(c) (bit 2 flipped by bit 3).  The swizzle is applied on the global
// side of the DMA, which writes each 1 KB load contiguously.
template <int JB, int SC, bool FB = false>
__global__ __launch_bounds__(512) void rank_z_lds(const RankZArgs args) {
    constexpr int D = SC / 32;                         // steps in flight = steps per slice
    constexpr int FBYTES = 16 * JB * SC * 2;           // one F slice
    constexpr int RPL = FB ? 32 / JB : 1024 / (2 * SC);   // F rows per 1 KB load
    constexpr int FLW = FB ? JB : 16 * JB / RPL / 8;   // F loads per wave per slice
    constexpr int ROWB = 32 * JB;                      // FB: bytes of one slice row
    static_assert(!FB || (SC == 256 && (JB == 1 || JB == 2 || JB == 4 || JB == 8)), "FB: whole rows per load");
    static_assert(FB || (FLW >= 1 && 16 * JB == FLW * 8 * RPL), "F slice is whole loads for 8 waves");
    static_assert(!FB || FLW * 8 * RPL == SC, "FB: the slice's rows are whole loads for 8 waves");
    static_assert(2 * FBYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t fs[2 * FBYTES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const RankZMember& a = args.mem[blockIdx.z];
    if ((int)blockIdx.y >= a.n_used) return;            // a member with fewer chunks than the grid
    const int M = args.M, C = a.C, ldy = args.ldy;
    const int m0 = (int)blockIdx.x * 128;
    const int m = m0 + wave * 16 + l16;
    const int cb = (int)blockIdx.y * a.chunk_c;
    const int ce = min(C, cb + a.chunk_c);
    const int nsl = (ce - cb + SC - 1) / SC;
    const int rl = args.rl;
    const __amdgpu_buffer_rsrc_t rsY = make_rsrc(a.Y + (size_t)m0 * ldy, strided_panel_bytes(M, m0, 128, C, ldy));
    const __amdgpu_buffer_rsrc_t rsF =
        FB ? make_rsrc(a.F, whole_bytes(C, args.f_ld)) : make_rsrc(a.F + (size_t)args.f_j0 * C, whole_bytes(rl, C));
    const uint32_t yoff = m < M ? (uint32_t)((m - m0) * ldy + cb + 8 * g4) * 2u : kOOB;
    // F slice: load i (1 KB) covers rows RPL i .. RPL i + RPL - 1; wave w issues i = FLW w ..
    auto fb_swz = [](int c) -> int {                   // JB >= 2: slot XOR for row c
        if constexpr (JB == 2) return (c >> 3) & 1;
        else if constexpr (JB == 4) return ((c >> 1) & 1) | (((c >> 3) & 1) << 1);
        else return (c & 3) | (((c >> 3) & 1) << 2);
    };
    auto fb_row = [](int c) -> int { return c ^ (((c >> 3) & 1) << 2); };   // JB = 1 (its own inverse)
    auto issue_f = [&](int sl, uint8_t* buf) {
#pragma unroll
        for (int t = 0; t < FLW; ++t) {
            const int i = wave * FLW + t;
            if constexpr (FB) {                        // slice row p, 16-byte piece q of the load's lane
                const int p = RPL * i + lane / (2 * JB), q = lane % (2 * JB);
                int row, j;
                if constexpr (JB == 1) {
                    row = fb_row(p);
                    j = 8 * q;
                } else {
                    row = p;
                    j = 16 * ((q >> 1) ^ fb_swz(p)) + 8 * (q & 1);
                }
                const int c = cb + sl * SC + row;
                const uint32_t off =
                    (c < ce && j < rl) ? (uint32_t)(c * args.f_ld + args.f_j0 + j) * 2u : kOOB;
                g2lds16<true>(rsF, buf + i * 1024, off);
            } else {
                const int row = RPL * i + lane / (SC / 8);
                const int col = cb + sl * SC + (((lane % (SC / 8)) ^ (row & 15)) << 3);
                const uint32_t off = (row < rl && col < ce) ? (uint32_t)(row * C + col) * 2u : kOOB;
                g2lds16<true>(rsF, buf + i * 1024, off);
            }
        }
    };
    auto ld = [&](int step) -> bf16x8 {
        const int c = cb + 32 * step + 8 * g4;
        const uint32_t o = (yoff == kOOB || c >= ce) ? kOOB : yoff + (uint32_t)(64 * step);
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsY, o, 0, 0));
    };
    f32x4 acc[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Y fragments two slices ahead (2 D loads of 16 bytes in flight per lane):
    // with one workgroup per CU, one slice ahead left ~64 KB in flight per CU,
    // about 2 us of the CU's share of HBM bandwidth.  yr[0 .. D) serves the
    // even slices, yr[D .. 2 D) the odd ones.  The slices run in pairs with
    // no branch inside (the count rounded up to even: past the chunk F and Y
    // read zeros and add nothing), so that the compiler's own waits before
    // each use keep every load of the other slices in flight.
    bf16x8 yr[2 * D];
    issue_f(0, fs);
#pragma unroll
    for (int u = 0; u < 2 * D; ++u) yr[u] = ld(u);
    vmcnt_le<2 * D>();                                 // this wave's part of slice 0 (older than the 2 D Y loads)
    __syncthreads();
    auto slice = [&](int sl, bf16x8* y) {
        const uint8_t* const fb = fs + (sl & 1) * FBYTES;
        issue_f(sl + 1, fs + ((sl + 1) & 1) * FBYTES);  // zeros past the chunk
#pragma unroll
        for (int u = 0; u < D; ++u) {
            bf16x8 ff[JB];
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if constexpr (FB) {                    // rows c = 32 u + 8 g4 + (0 .. 7), column jb 16 + l16
                    const int c = u * 32 + g4 * 8 + (l16 >> 2);   // bit 2 clear: c + 4 keeps fb_swz
                    if constexpr (JB == 1) {
                        const uint8_t* const p = fb + (l16 & 3) * 8;
                        ff[jb] = cat_tr(lds_tr4(p + fb_row(c) * ROWB), lds_tr4(p + fb_row(c + 4) * ROWB));
                    } else {
                        const uint8_t* const p = fb + c * ROWB + ((jb ^ fb_swz(c)) << 5) + (l16 & 3) * 8;
                        ff[jb] = cat_tr(lds_tr4(p), lds_tr4(p + 4 * ROWB));
                    }
                } else {
                    ff[jb] = lds_b128(fb + (jb * 16 + l16) * (SC * 2) + (((u * 4 + g4) ^ l16) << 4));
                }
            }
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) acc[jb] = mfma16(ff[jb], y[u], acc[jb]);
            y[u] = ld(sl * D + u + 2 * D);             // zeros past the chunk
        }
        vmcnt_le<D>();                                 // slice sl + 1's F and the Y loads older than this slice's D
        __syncthreads();
    };
    for (int sl = 0; sl < nsl; sl += 2) {
        slice(sl, yr);
        slice(sl + 1, yr + D);
    }
    vmcnt_le<0>();
    // lane holds Z^T rows j = 16 jb + 4 g4 + e at column m
    if (m < M) {
        if (a.row_scale) {
            const float rsc = a.row_scale[m];
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) acc[jb] *= rsc;
        }
        float* const out = a.out + (size_t)blockIdx.y * a.chunk_stride + (size_t)m * a.z_ld + a.z_j0;
        const bool vec = ((a.z_ld | a.z_j0) & 3) == 0;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            const int j = 16 * jb + 4 * g4;
            if (vec && j + 3 < rl) {
                *reinterpret_cast<f32x4*>(out + j) = acc[jb];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < rl) out[j + e] = acc[jb][e];
            }
        }
    }
}

// rank_stream side planes: hi(j, m) = bf16(Z[m][j]), lo(j, m) = bf16(Z[m][j] - hi),
// j < r, m < Mp (zero for m >= M), stored at e = zt_index(j, m, r); blockIdx.y
// selects one of two problems; the first one's rows may carry a scale (rs0).
// tiled = 1 (r >= 32): one workgroup per 128-token block and 32 rank rows, the
// block's Z rows read as whole 128-byte segments into LDS and written out as
// plane rows; otherwise one thread per plane element (reads r floats apart).
__device__ __forceinline__ void zt_hilo_put(uint16_t* hi, uint16_t* lo, size_t e, float v) {
    const __bf16 h = (__bf16)v;
    const __bf16 l = (__bf16)(v - (float)h);
    hi[e] = __builtin_bit_cast(uint16_t, h);
    lo[e] = __builtin_bit_cast(uint16_t, l);
}

__global__ __launch_bounds__(256) void zt_hilo(const float* __restrict__ z0, const float* __restrict__ z1,
                                               uint16_t* __restrict__ hi0, uint16_t* __restrict__ lo0,
                                               uint16_t* __restrict__ hi1, uint16_t* __restrict__ lo1, int M, int Mp,
                                               int r, const float* __restrict__ rs0, int tiled) {
    const float* z = blockIdx.y ? z1 : z0;
    uint16_t* const hi = blockIdx.y ? hi1 : hi0;
    uint16_t* const lo = blockIdx.y ? lo1 : lo0;
    const float* const rs = blockIdx.y ? nullptr : rs0;
    if (tiled) {
        __shared__ float tile[32 * 129];
        const int njt = (r + 31) / 32;
        const int tb = (int)blockIdx.x / njt, j0 = ((int)blockIdx.x % njt) * 32;
        const int m0 = tb * kSideBlock;
        const int t = threadIdx.x;
        // reads, all issued before the first LDS store: element i is
        // m = m0 + t / 32 + 8 i, j = j0 + t % 32
        // (buffer loads: rows past M and columns past r read zeros, no branch per load)
        const int j = j0 + (t & 31);
        const int rows = max(0, min(M - m0, kSideBlock));
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(z + (size_t)m0 * r, (uint64_t)rows * r * 4u);
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int ml = (t >> 5) + 8 * i;
            const uint32_t off = j < r ? (uint32_t)(ml * r + j) * 4u : kOOB;
            v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, off, 0, 0));
        }
        if (rs) {
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(rs + m0, (uint64_t)rows * 4u);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] *= __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      rr, (uint32_t)((t >> 5) + 8 * i) * 4u, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[(t & 31) * 129 + (t >> 5) + 8 * i] = v[i];
        __syncthreads();
        // writes: element i is j = j0 + t / 128 + 2 i, m = m0 + t % 128
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int jl = (t >> 7) + 2 * i, jj = j0 + jl;
            if (jj < r) zt_hilo_put(hi, lo, zt_index(jj, m0 + (t & 127), r), tile[jl * 129 + (t & 127)]);
        }
        return;
    }
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)r * Mp) return;
    const int64_t blk = e / ((int64_t)r * kSideBlock);
    const int rem = (int)(e - blk * r * kSideBlock);
    const int j = rem / kSideBlock;
    const int64_t m = blk * kSideBlock + rem % kSideBlock;
    const float v = m < M ? z[(size_t)m * r + j] * (rs ? rs[m] : 1.f) : 0.f;
    zt_hilo_put(hi, lo, (size_t)e, v);
}

// F^T rows for the Z-mode pass over dY: out[j][n] = B[n][j].
// Every member of a group in one launch: member m's B^T [r][N_m] (rows n0[m] ..
// n0[m + 1] - 1 of B) at out + r n0[m], the members side by side.
struct TransposeRankArgs {
    int n0[kMaxMembers + 1];
    int G, r;
};

__global__ __launch_bounds__(256) void transpose_rank(const uint16_t* __restrict__ B, uint16_t* __restrict__ out,
                                                      const TransposeRankArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)a.r * a.n0[a.G]) return;
    int m = 0;                                          // member whose block holds e
#pragma unroll
    for (int k = 1; k < kMaxMembers; ++k) m += (k < a.G && e >= (int64_t)a.r * a.n0[k]) ? 1 : 0;
    const int64_t loc = e - (int64_t)a.r * a.n0[m];
    const int nm = a.n0[m + 1] - a.n0[m];
    const int j = (int)(loc / nm), n = a.n0[m] + (int)(loc % nm);
    out[e] = B[(size_t)n * a.r + j];
}

// out[m * out_ld + out_j0 + j] = sum over k < n_parts of part[k * M * w + m * w + j]
// (j < w), added in increasing k: the contraction-chunk partials of one
// rank_z_lds launch (compact rows of w columns) into its columns of Z, for
// member blockIdx.y of the launch (members with one chunk wrote Z themselves).
// Each thread owns 4 consecutive partial elements; the partial loads are
// issued 8 at a time so that their latencies overlap (the additions keep the
// fixed order).
struct PartialSumArgs {
    const float* part[kMaxMembers];
    const float* row_scale[kMaxMembers];
    int out_j0[kMaxMembers];
    int n_parts[kMaxMembers];
    float* out;
    int M, w, out_ld;
};

__global__ __launch_bounds__(256) void partial_sum(const PartialSumArgs args) {
    const int mem = blockIdx.y;
    const int n_parts = args.n_parts[mem];
    if (n_parts <= 1) return;
    const float* __restrict__ const part = args.part[mem];
    const float* __restrict__ const row_scale = args.row_scale[mem];
    float* __restrict__ const out = args.out;
    const int M = args.M, w = args.w, out_ld = args.out_ld, out_j0 = args.out_j0[mem];
    const int64_t n = (int64_t)M * w;
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e0 >= n) return;
    const int cnt = (int)min<int64_t>(4, n - e0);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    auto load4 = [&](int k) -> f32x4 {
        const float* p = part + (size_t)k * n + e0;
        if (cnt == 4 && (n & 3) == 0) return *reinterpret_cast<const f32x4*>(p);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < cnt; ++i) v[i] = p[i];
        return v;
    };
    int k = 0;
    for (; k + 8 <= n_parts; k += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = load4(k + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < n_parts; ++k) s += load4(k);
    for (int i = 0; i < cnt; ++i) {
        const int64_t e = e0 + i;
        const int64_t mm = e / w;
        out[mm * out_ld + out_j0 + (e - mm * w)] = row_scale ? s[i] * row_scale[mm] : s[i];
    }
}

// Final adapter gradients from the rank_stream partials:
//   dA[j][k] = s * sum_chunk GA[chunk][k][j]   ([ra][K] output; ra = G r for a group)
//   dB[n][j] = s * sum_chunk GB[chunk][n][j]   ([N][rb] output)
// in the tensor dtype, overwritten or accumulated.
struct GradFinalArgs {
    const float* ga;        // [n_chunk][K][ra]
    const float* gb;        // [n_chunk][N][rb]
    void* dA;               // [ra][K]
    void* dB;               // [N][rb]
    int K, N, ra, rb, n_chunk;
    float s;
    int f32_out, accumulate;
    const uint16_t* a_col_scale;   // optional bf16 scale of dA's column k (the RMSNorm weight g)
    int tiled;                     // dA through LDS tiles (blocks before the element blocks)
};

// tiled = 1 (ra >= 64): dA in tiles of 64 k x 64 j, one workgroup each, through
// LDS, so that the partial reads (rows of j) and the transposed dA writes (rows
// of k) are whole segments instead of one 2-byte write per line; the element
// blocks after them then cover dB alone.  Every element adds its chunks in the
// same order either way.
__device__ __forceinline__ void grad_store(const GradFinalArgs& a, void* dst, size_t o, float v) {
    if (a.f32_out) {
        float* p = reinterpret_cast<float*>(dst);
        if (a.accumulate) v += p[o];
        p[o] = v;
    } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(dst);
        if (a.accumulate) v += bf16_bits_to_f32(p[o]);
        p[o] = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
}

__global__ __launch_bounds__(256) void grad_final(const GradFinalArgs a) {
    __shared__ float tile[64 * 65];
    const int64_t na = (int64_t)a.K * a.ra, nb = (int64_t)a.N * a.rb;
    const int nkt = (a.K + 63) / 64;
    const int nta = a.tiled ? nkt * ((a.ra + 63) / 64) : 0;
    if ((int)blockIdx.x < nta) {
        const int k0 = ((int)blockIdx.x % nkt) * 64, j0 = ((int)blockIdx.x / nkt) * 64;
        const int lo = threadIdx.x & 63, hi = threadIdx.x >> 6;
        // sums: element i of the thread is k = k0 + hi + 4 i, j = j0 + lo
        const int j = j0 + lo;
        float acc[16];
        size_t off[16];
        bool ok[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = k0 + hi + 4 * i;
            ok[i] = j < a.ra && k < a.K;
            off[i] = ok[i] ? (size_t)k * a.ra + j : 0;
            acc[i] = 0.f;
        }
        int c = 0;
        for (; c + 2 <= a.n_chunk; c += 2) {        // two chunks of loads in flight, added in chunk order
            float v0[16], v1[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v0[i] = ok[i] ? a.ga[(size_t)c * na + off[i]] : 0.f;
                v1[i] = ok[i] ? a.ga[(size_t)(c + 1) * na + off[i]] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] += v0[i];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] += v1[i];
        }
        for (; c < a.n_chunk; ++c) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] += ok[i] ? a.ga[(size_t)c * na + off[i]] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kl = hi + 4 * i;
            float v = acc[i] * a.s;
            if (a.a_col_scale && ok[i]) v *= bf16_bits_to_f32(a.a_col_scale[k0 + kl]);
            tile[lo * 65 + kl] = v;
        }
        __syncthreads();
        // stores: element i is j = j0 + hi + 4 i, k = k0 + lo
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int jl = hi + 4 * i, jj = j0 + jl, k = k0 + lo;
            if (jj < a.ra && k < a.K) grad_store(a, a.dA, (size_t)jj * a.K + k, tile[jl * 65 + lo]);
        }
        return;
    }
    const int64_t e = ((int64_t)blockIdx.x - nta) * 256 + threadIdx.x + (a.tiled ? na : 0);
    if (e >= na + nb) return;
    const bool isA = e < na;
    const int64_t f = isA ? e : e - na;
    const int64_t n = isA ? na : nb;
    const float* part = isA ? a.ga : a.gb;
    float sum = 0.f;
    int k = 0;
    for (; k + 8 <= a.n_chunk; k += 8) {       // eight loads in flight, summed in chunk order
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(k + u) * n + f];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; k < a.n_chunk; ++k) sum += part[(size_t)k * n + f];
    float v = sum * a.s;
    size_t o;
    if (isA) {
        const int kk = (int)(f / a.ra), j = (int)(f % a.ra);
        o = (size_t)j * a.K + kk;
        if (a.a_col_scale) v *= bf16_bits_to_f32(a.a_col_scale[kk]);
    } else {
        o = (size_t)f;
    }
    grad_store(a, isA ? a.dA : a.dB, o, v);
}

}  // namespace lora
