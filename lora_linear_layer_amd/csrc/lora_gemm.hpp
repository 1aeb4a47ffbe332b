// Fused LoRA GEMM for gfx950: 8 waves, direct global->LDS staging, fragment
// reads software-pipelined against the MFMAs, transposed LDS reads for the
// input-gradient operand.
//
// One kernel computes
//   Out[p][q] = sum_c L[p][c] R(q, c)  +  s * sum_j E(q, j) Z[p][j]
//   Z[p][j]   = sum_c L[p][c] F(j, c)      (rank-r product, formed on chip)
// which is both directions of the LoRA linear layer:
//   forward (page "ms-swift高效微调组合：LoRA+UnSloth提速实践", section 1.2
//     "算子融合": Linear, LoRA_A, LoRA_B and the add in one launch):
//     P=M, Q=N, C=K, L=X, R(q,c)=W[q][c], F(j,c)=A[j][c], E(q,j)=B[q][j], Z=U.
//   input gradient (page "Unsloth — 微调 2-5x 加速", section "核心要点",
//     item 2: (A B) dY is evaluated as A (B dY), only rank-r intermediates):
//     P=M, Q=K, C=N, L=dY, R(q,c)=W[c][q], F(j,c)=B[c][j], E(q,j)=A[j][q], Z=V.
//
// Work split: a 256 (p) x 256 (q) output tile per workgroup of 8 waves,
// 2 (p) x 4 (q); each wave owns 128 p x 64 q = 8 x 4 MFMA 16x16x32 tiles
// (128 fp32 accumulators per lane), two waves per SIMD.
//
// Pipeline: the contraction advances 64 at a time through two LDS stages
// (L 32 KB, R 32 KB, F RPAD x 128 B).  Stage kt + 2 is fetched with
// buffer_load ... lds (global memory straight into LDS, no VGPRs) into the slot
// stage kt just vacated.  Each stage is two 32-wide steps; the fragments of the
// next step are read from LDS while the MFMAs of the current step run, and the
// workgroup barrier sits between the two steps of a stage:
//   [step kk0: MFMA(frags A) | read frags B for kk1]
//   wait own loads of stage kt+1, barrier, issue loads of stage kt+2
//   [step kk1: MFMA(frags B) | read frags A for kk0 of stage kt+1]
// Out-of-range rows and contraction chunks get a buffer offset past the
// descriptor's range, which the hardware answers with zeros.
//
// LDS layouts:
//   contraction-contiguous tiles (L; R in forward; F in forward): rows of 64
//     values (128 B); 16-byte chunk ch of row x stored at chunk ch ^ (x & 7),
//     so the 8 lanes of each quarter of a fragment read hit distinct banks.
//   R in the input gradient: W rows c (512 B = 256 q), 32-byte slot s of row
//     c at slot s ^ sw512(c); fragments are gathered with ds_read_b64_tr_b16,
//     which hands each lane 4 values down a column.
// r <= 16: the rank-r product Z^T = F L^T reuses the L fragments already in
// registers; the 4 waves that share a p half each form Z for 32 of its 128
// rows.  The forward's F = A rows go to LDS like L; the input gradient's
// F (r = 8 or 16) arrives as B's own [c][j] rows and is read with the
// transposing LDS load, like the W tile.  In
// the epilogue Z meets in LDS and s Z E^T is applied with MFMA, s Z split into
// bf16 hi + lo halves that fill the two halves of the 32-long contraction.
// ZIN = true takes a precomputed Z [P][r] float32 instead (large r).
//
// Q4 = true: R is a 4-bit weight matrix (page "Unsloth — 微调 2-5x 加速",
// section "核心要点", item 3).  Its codes and absmax travel through registers
// instead of the direct LDS path: each thread loads 16 code bytes (32 weights
// of one row inside one 64-block) and that block's absmax when the stage is
// issued, and one step later decodes them, codebook[code] * absmax in float32
// rounded to bf16 (the standalone dequantisation's exact values; the 16
// possible values of a block are formed once per lane pair and looked up in
// registers), into
// the stage's R tile in the same swizzled layout, before the barrier that
// publishes the stage.  Every weight is decoded once per workgroup; the
// reads, MFMAs and epilogue are the 16-bit kernel's.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "ranges.hpp"

namespace lora {

typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxMembers = 8;      // linears sharing one input in one grouped call
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;

constexpr uint32_t kOOB = 0x80000000u;        // buffer offset beyond every range -> zeros
constexpr int32_t kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes > kMaxRange ? kMaxRange : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

// A range known to be below 2^31 bytes (32-bit arithmetic, no clipping).  Base
// and range are uniform; passing them through readfirstlane says so, which
// keeps the compiler from wrapping the loads in a per-lane descriptor loop
// when it has kept a uniform address in vector registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void* base, int bytes) {
    const uint64_t b = (uint64_t)(size_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void* const ub = (void*)(size_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// 16 bytes per lane from global (rsrc + voff) into LDS at lds_wave_base + 16 * lane.
// UNTRACKED = true issues it as asm, hidden from the compiler's wait-count
// bookkeeping: the compiler cannot tell a transposing LDS read
// (ds_read_b64_tr_b16) from an in-flight load into another stage and would
// put a full vmcnt(0) in front of every such read, exposing the next stage's
// load latency on every step.  Callers wait for these loads themselves
// (vmcnt_le) before the barrier that publishes a stage.  M0 carries the
// wave's LDS base.
template <bool UNTRACKED = false>
__device__ __forceinline__ void g2lds16(__amdgpu_buffer_rsrc_t rs, void* lds_wave_base, uint32_t voff) {
    if constexpr (UNTRACKED) {
        const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void_ptr)lds_wave_base);
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)lds_wave_base, 16, voff, 0, 0, 0);
    }
}

// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element j % 4
// of the 8-byte rows addressed by lanes j / 4, 4 + j / 4, 8 + j / 4, 12 + j / 4.
__device__ __forceinline__ i16x4 lds_tr4(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p);
}

__device__ __forceinline__ bf16x8 cat_tr(const i16x4& lo, const i16x4& hi) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 lds_b128(const void* p) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int sw512(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vmcnt_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Workgroup barrier that orders LDS traffic only (no wait on global loads).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct GemmArgs {
    const uint16_t* L;      // [P][C] bf16
    const uint16_t* R;      // forward: [Q][C]; input gradient: [C][Q]
    const uint8_t* Rq;      // 4-bit weights: codes, forward [Q][C/2], input gradient [C][Q/2]
    const uint16_t* Rabs;   // 4-bit weights: fp16 absmax, forward [Q][C/64], input gradient [C][Q/64]
    const float* codebook;  // 4-bit weights: 16 float32 values
    const uint16_t* F;      // forward: A [r][C]; input gradient: B [C][r]
    const uint16_t* E;      // forward: B [Q][r]; input gradient: A [r][Q]
    const float* Zin;       // precomputed Z [P][r] (ZIN), else unused
    uint16_t* Out;          // [P][Q] bf16
    float* Zsave;           // [P][r] float32 or nullptr (each row by one workgroup of its row panel)
    float* Part;            // split contraction: float32 partial tiles [split][tile - first_split][256][256]
    // Input gradient, in-tile Z only: the bf16 planes hi = bf16(Z^T), lo = bf16(Z^T - hi) of
    // Z = V and of U (read from Uin [P][r] float32), [r][Mp] in the token-block-major order of
    // zt_index, tokens p >= P zero; written (each row by one workgroup of its row panel) for the
    // adapter-gradient pass, or not at all when Zt_hi is nullptr
    uint16_t *Zt_hi, *Zt_lo, *Ut_hi, *Ut_lo;
    const float* Uin;
    int Mp;
    int P, Q, C, r;
    int first_split, split, kc;   // split contraction: first split tile, slices, 64-wide stages per slice
    float s;
    // Precomputed Z: its rows are z_ld floats.  Output columns q in [member_q0[i],
    // member_q0[i + 1]) belong to member i, whose rank term uses Z columns i r ..
    // i r + r - 1 (linears sharing one input, forward); a plain layer is one member.
    int z_ld;
    int n_members;
    int member_q0[kMaxMembers + 1];
    // Optional per-row scale (RMSNorm in front of the layer: 1 / rms of each
    // input row).  Forward: every output row after the rank-r term and the
    // saved Z.  Input gradient: only the V planes written for the adapter
    // gradients (the output is scaled by the row kernel that follows).
    // nullptr: none.
    const float* row_scale;
};

namespace g2 {
constexpr int BP = 256, BQ = 256, BK = 64;
constexpr int TILE = BP * BK * 2;             // 32 KB per operand per stage
}  // namespace g2

// Wave layout of the 256 x 256 tile: 2 (p) x 4 (q) waves of 128 x 64, two
// waves per SIMD.
namespace g2w {
constexpr int NT = 512;
constexpr int WQN = 4;        // waves along q
constexpr int QB = 4;         // q blocks of 16 per wave
constexpr int ZB = 2;         // p blocks per wave in the rank-r product
constexpr int LPW = 4;        // 1 KB loads per wave per operand per stage
}  // namespace g2w

template <int RPAD, bool ZIN, bool Q4 = false>
struct GemmSmem {
    static constexpr int F_BYTES = ZIN ? 0 : RPAD * g2::BK * 2;
    static constexpr int STAGE = 2 * g2::TILE + F_BYTES;
    static constexpr int LUT = 2 * STAGE;                       // 4-bit codebook (16 float32)
    static constexpr int TOTAL = 2 * STAGE + (Q4 ? 64 : 0);
    static_assert(F_BYTES % 1024 == 0, "F tile is whole 1 KB wave loads");
    static_assert(ZIN || g2::BP * RPAD * 4 <= TOTAL, "Z exchange must fit");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <int JT, int QB>
struct Frags {
    bf16x8 r[QB];     // R, QB q blocks of 16
    bf16x8 l[8];      // L, 8 p blocks of 16 (slot i = block (i + ZROT wq) % 8)
    bf16x8 f[JT];     // F, rank rows
};

// 4-bit decode in registers.  The 16 values bf16(codebook[n] * absmax) of one
// absmax block are formed once per lane pair (float32 products, rounded as
// when each weight's product is formed on its own) and kept as byte tables:
// low bytes in lb, high bytes in hb, four entries per register.  The two lanes
// of an even / odd pair decode the same block: each forms one 8-entry half
// (the even lane codes 0..7, the odd lane codes 8..15) and takes the other
// half from its partner with a DPP swap, so lb / hb[0..1] hold the lane's own
// half and [2..3] the partner's.  v_perm_b32 looks up four codes per
// instruction in each half, and one more picks the half by bit 3 of each code
// (cl flips that choice on odd lanes).  This replaces one LDS read of the
// codebook per weight, which held both 4-bit GEMMs back by about 12 %; sharing
// the table removes 20 of the ~200 VALU instructions per stage and lane.
struct Q4Lut {
    uint32_t lb[4], hb[4];
    uint32_t cl;        // 0x03020100 (even lane), 0x07060504 (odd lane)
};

// byte i of the result = byte sel_i (0 .. 7) of the 8-byte value {hi : lo}
__device__ __forceinline__ uint32_t vperm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Every lane of the wave must call this (the swap reads the partner lane).
__device__ __forceinline__ Q4Lut q4_lut(const float* lut, float am, int odd, uint32_t cl) {
    Q4Lut t;
    t.cl = cl;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(lut + 8 * odd + 4 * g);
        const uint32_t t01 = pack_bf16x2(v[0] * am, v[1] * am), t23 = pack_bf16x2(v[2] * am, v[3] * am);
        t.lb[g] = vperm(t23, t01, 0x06040200u);
        t.hb[g] = vperm(t23, t01, 0x07050301u);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {       // quad_perm [1, 0, 3, 2]: swap with lane ^ 1
        t.lb[2 + g] = (uint32_t)__builtin_amdgcn_mov_dpp((int)t.lb[g], 0xB1, 0xF, 0xF, false);
        t.hb[2 + g] = (uint32_t)__builtin_amdgcn_mov_dpp((int)t.hb[g], 0xB1, 0xF, 0xF, false);
    }
    return t;
}

// One code dword (byte k: code 2k in the low nibble, code 2k + 1 in the high
// one) -> o[k] = the bf16 pair of codes 2k, 2k + 1.
__device__ __forceinline__ void q4_decode8(const Q4Lut& t, uint32_t q, uint32_t* o) {
    const uint32_t ln = q & 0x0F0F0F0Fu, hn = (q >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t n = vperm(hn, ln, h ? 0x07030602u : 0x05010400u);   // codes 4h .. 4h + 3, one per byte
        const uint32_t sel = n & 0x07070707u;
        // byte i: i for codes in the lane's own half, i + 4 for the partner's
        const uint32_t half = ((n >> 1) & 0x04040404u) ^ t.cl;
        const uint32_t lo = vperm(vperm(t.lb[3], t.lb[2], sel), vperm(t.lb[1], t.lb[0], sel), half);
        const uint32_t hi = vperm(vperm(t.hb[3], t.hb[2], sel), vperm(t.hb[1], t.hb[0], sel), half);
        o[2 * h] = vperm(hi, lo, 0x05010400u);
        o[2 * h + 1] = vperm(hi, lo, 0x07030602u);
    }
}

// SPLIT = true (precomputed Z only): tiles below first_split run whole; the
// others run as `split` workgroups each, slice v covering the contraction
// stages [kc v, kc (v + 1)), storing a float32 partial tile (slice 0 with the
// rank-r term) that split_finish adds in order and rounds to bf16.  Used when
// the output has too few tiles to fill the chip (e.g. d_out = 1024: all tiles
// split) and for the tiles of a last, partly empty round.
template <bool TRANS, int RPAD, bool ZIN, bool Q4 = false, bool SPLIT = false, bool RT = false>
__global__ __launch_bounds__(g2w::NT) void lora_gemm(const GemmArgs a) {
    using namespace g2;
    using namespace g2w;
    // R rows along q, contiguous in c ([Q][C]): the forward's W, and the input
    // gradient's when it is given as W^T (RT); otherwise the input gradient's W
    // is [C][Q] and its fragments are gathered with transposing LDS reads
    constexpr bool RQC = !TRANS || RT;
    static_assert(!(RT && (Q4 || !TRANS)), "RT: 16-bit input-gradient weights only");
    using SM = GemmSmem<RPAD, ZIN, Q4>;
    static_assert(ZIN || !Q4, "4-bit GEMMs take Z precomputed");
    static_assert(!SPLIT || ZIN, "split contraction: precomputed Z");
    constexpr int JT = ZIN ? 1 : RPAD / 16;
    // L fragment slot i holds p block (i + ZROT wq) % 8: with the rank-r product
    // formed in the tile, slots 0 .. ZB - 1 are the wave's own Z blocks; with Z
    // precomputed the order is plain, so every fragment read has a constant offset
    constexpr int ZROT = ZIN ? 0 : ZB;
    constexpr int F_LOADS = SM::F_BYTES / 1024;   // done by waves 0 .. F_LOADS - 1
    static_assert(F_LOADS <= 8, "F tile larger than one load per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SM::TOTAL];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // uniform per wave: keeps the wave-dependent parts of the LDS and global
    // offsets in scalar registers (fewer VGPRs, no spills in most variants)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wp = wave / WQN, wq = wave % WQN;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int P = a.P, Q = a.Q, C = a.C, r = a.r;
    const int nPt = (P + BP - 1) / BP, nQt = (Q + BQ - 1) / BQ;
    int pt, qt, kbase = 0, slice = -1, stile = 0;   // slice -1: whole tile
    if constexpr (SPLIT) {
        // whole tiles first, then the slices, each set spread evenly over the
        // XCDs on its own (one mapping over both gave some XCDs only whole
        // tiles and others only slices)
        const int T = nPt * nQt, b = blockIdx.x;
        int tile;
        if (b < a.first_split) {
            tile = xcd_contiguous(b, a.first_split);
        } else {
            const int v = xcd_contiguous(b - a.first_split, (T - a.first_split) * a.split);
            stile = v / a.split;
            slice = v % a.split;
            kbase = slice * a.kc;
            tile = a.first_split + stile;
        }
        grouped_tile<4>(tile, nPt, nQt, pt, qt);
    } else {
        grouped_tile<4>(xcd_contiguous(blockIdx.x, nPt * nQt), nPt, nQt, pt, qt);
    }
    const int p0 = pt * BP, q0 = qt * BQ;

    // ------------------------------------------------------------ load plan
    // Row layout tiles: load i of wave w covers rows (LPW w + i) * 8 + lane / 8;
    // lane's 16-byte chunk is (lane % 8) ^ (row % 8) = (lane % 8) ^ (lane / 8),
    // the same for every i, so one base offset plus a uniform stride suffices.
    const int kc_row0 = wave * LPW * 8 + (lane >> 3);
    const int kc_ch = ((lane & 7) ^ (lane >> 3)) * 8;
    const __amdgpu_buffer_rsrc_t rsL = make_rsrc(a.L + (size_t)p0 * C, panel_bytes(P, p0, BP, C));
    const uint32_t offL = (uint32_t)(kc_row0 * C + kc_ch) * 2u;
    __amdgpu_buffer_rsrc_t rsR;
    uint32_t offR = 0;
    int chR[LPW == 8 ? 4 : 2] = {};
    if constexpr (Q4) {
        // R tiles come through registers (load_q / decode_q)
    } else if constexpr (RQC) {
        rsR = make_rsrc(a.R + (size_t)q0 * C, panel_bytes(Q, q0, BQ, C));
        offR = (uint32_t)(kc_row0 * C + kc_ch) * 2u;
    } else {
        // W rows c (512 bytes each); load i of wave w covers rows
        // 2 (LPW w + i) + lane / 32.  The slot swizzle sw512 of those rows
        // depends on i only through i % 2 (and i / 4 when LPW = 8).
        const int pch = lane & 31, h = lane >> 5;
        const int row0 = wave * 2 * LPW + h;
#pragma unroll
        for (int v = 0; v < (LPW == 8 ? 4 : 2); ++v) {
            const int row = row0 + 2 * (v & 1) + 8 * (v >> 1);
            chR[v] = (((pch >> 1) ^ sw512(row)) * 2 + (pch & 1)) * 8;   // q offset inside the tile
        }
        offR = (uint32_t)(row0 * Q) * 2u;
    }
    __amdgpu_buffer_rsrc_t rsF;
    uint32_t offF = kOOB;
    int fch = 0, frow = 0;
    if constexpr (!ZIN) {
        rsF = make_rsrc(a.F, TRANS ? whole_bytes(C, r) : whole_bytes(r, C));   // B [C][r] or A [r][C]
        frow = wave * 8 + (lane >> 3);                       // j (waves 0 .. RPAD/8 - 1)
        fch = kc_ch;
        offF = (uint32_t)(frow * C + fch) * 2u;
    }

    // 4-bit weights: each thread fetches 16 bytes of codes (32 weights of one
    // row, within one 64-block) and the block's absmax per unit into
    // registers when a stage is issued, and decodes them into the stage's bf16
    // R tile (same LDS layout as the 16-bit path) before the barrier that
    // publishes it.  512 units per stage, 512 / NT per thread.
    constexpr int QU = Q4 ? 512 / NT : 1;
    u32x4 qreg[QU];
    uint32_t am_reg[QU];      // fp16 bits: converted at decode, so the load is not waited for at issue
#pragma unroll
    for (int u = 0; u < QU; ++u) { qreg[u] = u32x4{0u, 0u, 0u, 0u}; am_reg[u] = 0u; }
    if constexpr (Q4) {
        if (tid < 16) reinterpret_cast<float*>(smem + SM::LUT)[tid] = a.codebook[tid];
    }
    // Forward 4-bit codes [Q][C/2]: a stage is 32 bytes of each weight row, half
    // of a 64-byte request, so the codes of two stages are fetched together as
    // one 64-byte run per row (pieces 0, 1: the even stage; 2, 3: the odd one).
    // Lane l of wave w takes piece l % 4 of row 16 w + l / 4 and piece
    // (l % 4 + 2) % 4 of the row 128 below: one piece of each stage, so each
    // stage's decode stays one 16-byte piece per lane.
    static_assert(!Q4 || TRANS || (NT == 512 && QU == 1), "paired code loads: 512 threads");
    const int qrA = wave * 16 + (lane >> 2), qrB = qrA + 128;
    const int qp1 = lane & 3, qp2 = (qp1 + 2) & 3;
    u32x4 qregB = {0u, 0u, 0u, 0u};
    uint32_t amB = 0u;
    // Forward codes and absmax come through buffer resources built per stage
    // (scalar work) on the stage's first byte of the panel's 256 rows, so each
    // lane's offsets stay constant and rows past the weight's end read zeros;
    // the odd stage's pieces of the last row past C read zeros too, and a stage
    // past C elsewhere is fetched but never decoded.  (The input gradient keeps
    // plain loads: the same change made its loop slower.)
    uint32_t qoffA = 0, qoffB = 0, aoffA = 0, aoffB = 0;
    if constexpr (Q4 && !TRANS) {
        qoffA = (uint32_t)(qrA * (C >> 1) + 16 * qp1);
        qoffB = (uint32_t)(qrB * (C >> 1) + 16 * qp2);
        aoffA = (uint32_t)(qrA * (C >> 6) + (qp1 >> 1)) * 2u;
        aoffB = (uint32_t)(qrB * (C >> 6) + (qp2 >> 1)) * 2u;
    }
    auto load_q = [&](int kt0) {
        const int kt = kbase + kt0;              // stage of the whole contraction
        const int c0 = kt * BK;
        if constexpr (!TRANS) {
            if (kt0 & 1) return;                 // fetched with the even stage before it
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc32(a.Rq + (size_t)q0 * (C >> 1) + (c0 >> 1), q4_code_bytes(Q, q0, BQ, C, c0));
            const __amdgpu_buffer_rsrc_t ra =
                make_rsrc32(a.Rabs + (size_t)q0 * (C >> 6) + (c0 >> 6), q4_absmax_bytes(Q, q0, BQ, C, c0));
            qreg[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)qoffA, 0, 0);
            am_reg[0] = __builtin_amdgcn_raw_buffer_load_b16(ra, (int)aoffA, 0, 0);
            qregB = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)qoffB, 0, 0);
            amB = __builtin_amdgcn_raw_buffer_load_b16(ra, (int)aoffB, 0, 0);
            return;
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int unit = tid + u * NT;
            {                                // codes [C][Q/2]: row c = unit / 8, weights q0 + 32 (unit % 8) ..
                const int c = unit >> 3, pp = unit & 7;
                const bool ok = c0 + c < C && q0 + 32 * pp < Q;
                const size_t qq = (size_t)q0 + 32 * pp;
                qreg[u] = ok ? *reinterpret_cast<const u32x4*>(a.Rq + (size_t)(c0 + c) * (Q >> 1) + (qq >> 1))
                             : u32x4{0u, 0u, 0u, 0u};
                am_reg[u] = ok ? (uint32_t)a.Rabs[(size_t)(c0 + c) * (Q >> 6) + (qq >> 6)] : 0u;
            }
        }
    };
    // lanes l and l ^ 1 decode the same absmax block in both directions (the
    // same row and stage; the input gradient's 64-wide q block) and share its table
    const int q4odd = lane & 1;
    const uint32_t q4cl = q4odd ? 0x07060504u : 0x03020100u;
    auto decode_q = [&](int kt) {
        uint8_t* const Rs = smem + (kt & 1) * SM::STAGE + TILE;
        const float* const lut = reinterpret_cast<const float*>(smem + SM::LUT);
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int unit = tid + u * NT;
            // code dword d = 8 weights = 16-byte output chunk d.  Input gradient:
            // lanes with pp & 4 take their chunks in the order 1, 0, 3, 2, so that
            // each 16-byte store instruction of a row's 8 lanes covers both
            // halves of 4 slots (8 distinct bank groups) instead of one half of
            // 8 slots, of which the swizzle leaves 4 distinct
            u32x4 qv = qreg[u];
            uint32_t amb = am_reg[u];
            int fq = 0, fh = 0;                // forward: the row and half (stage piece) this lane decodes
            if constexpr (!TRANS) {
                const bool useA = (qp1 < 2) == ((kt & 1) == 0);
                if (!useA) { qv = qregB; amb = amB; }
                fq = useA ? qrA : qrB;
                fh = (useA ? qp1 : qp2) & 1;
            }
            const float am = f16_bits_to_f32((uint16_t)amb);
            const int sh = TRANS ? (unit >> 2) & 1 : 0;
            if (TRANS && sh) qv = u32x4{qv[1], qv[0], qv[3], qv[2]};
            const Q4Lut tab = q4_lut(lut, am, q4odd, q4cl);
            u32x4 outv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {    // code dword i -> output chunk i (8 weights)
                uint32_t o[4];
                q4_decode8(tab, qv[i], o);
                outv[i] = u32x4{o[0], o[1], o[2], o[3]};
            }
            if constexpr (!TRANS) {          // row q, 16-byte chunks 4h .. 4h + 3, chunk ch at ch ^ (q & 7)
                const int q = fq, hh = fh;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4*>(Rs + q * 128 + (((4 * hh + i) ^ (q & 7)) << 4)) = outv[i];
            } else {                         // row c, 32-byte slots 2 pp, 2 pp + 1 (swizzled by sw512)
                const int c = unit >> 3, pp = unit & 7;
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // outv[i] is chunk i ^ sh: slot 2 pp + i / 2, half (i & 1) ^ sh
                    const int slot = 2 * pp + (i >> 1);
                    *reinterpret_cast<u32x4*>(Rs + c * 512 + ((slot ^ sw512(c)) << 5) + ((i & 1) ^ sh) * 16) =
                        outv[i];
                }
            }
        }
    };

    // L and R of stage kt (R from the codes when Q4).  With on = false every
    // offset is out of range: the instructions still issue (keeping the loop
    // free of branches) and write zeros into the slot of stage kt, which no
    // later read uses.
    auto issue_lr = [&](int kt, bool on) {
        const int c0 = (kbase + kt) * BK;
        uint8_t* const Ls = smem + (kt & 1) * SM::STAGE;
        uint8_t* const Rs = Ls + TILE;
        // one per-lane base per operand and stage (or the out-of-range marker,
        // which stays out of range with any of the row increments added: they
        // are below 2^31), plus a uniform row increment per load
        const bool lok = on && c0 + kc_ch < C;
        const uint32_t vL = lok ? offL + (uint32_t)c0 * 2u : kOOB;
#pragma unroll
        for (int i = 0; i < LPW; ++i) g2lds16<TRANS>(rsL, Ls + (wave * LPW + i) * 1024, vL + (uint32_t)(i * 8 * C) * 2u);
        if constexpr (Q4) {
            load_q(kt);
        } else if constexpr (RQC) {
            const uint32_t vR = lok ? offR + (uint32_t)c0 * 2u : kOOB;
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                g2lds16<TRANS>(rsR, Rs + (wave * LPW + i) * 1024, vR + (uint32_t)(i * 8 * C) * 2u);
        } else {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.R + (size_t)c0 * Q + q0, gemm_wt_stage_bytes(C, Q, c0, q0));
            uint32_t vR[LPW == 8 ? 4 : 2];
#pragma unroll
            for (int v = 0; v < (LPW == 8 ? 4 : 2); ++v)
                vR[v] = (on && q0 + chR[v] < Q) ? offR + (uint32_t)chR[v] * 2u : kOOB;
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                g2lds16<TRANS>(rs, Rs + (wave * LPW + i) * 1024,
                               vR[(i & 1) | (LPW == 8 ? ((i >> 2) & 1) << 1 : 0)] + (uint32_t)(2 * i * Q) * 2u);
        }
    };
    // F of the rank-r product, straight from global memory into LDS in both
    // directions (waves 0 .. F_LOADS - 1, one 1 KB load each per stage).
    // Forward: A [r][C] rows are contiguous in c: rows j of 64 c, swizzled like L.
    // Input gradient (r = 8 or 16): B [C][r] rows are contiguous in j and land
    // as they are, [64 c][16 j] rows of 32 bytes, row c at physical row
    // c ^ 4 (c & 8 ? 1 : 0) so that the two 16-lane groups of a transposing
    // read (rows 8 apart) use different banks; lane l of wave w carries
    // physical row 32 w + l / 2, half l % 2 (j 8 h .. 8 h + 7; zeros when r = 8
    // and h = 1), and the fragments are gathered down the columns with
    // ds_read_b64_tr_b16 like the W tile.
    auto issue_f = [&](int kt) {
        if constexpr (!ZIN && !TRANS) {
            const int c0 = kt * BK;
            uint8_t* const Fs = smem + (kt & 1) * SM::STAGE + 2 * TILE;
            if (wave < F_LOADS)
                g2lds16<TRANS>(rsF, Fs + wave * 1024, (frow < r && c0 + fch < C) ? offF + (uint32_t)c0 * 2u : kOOB);
        } else if constexpr (!ZIN) {
            static_assert(RPAD == 16, "input-gradient in-tile F is 16 rank columns");
            const int c0 = kt * BK;
            uint8_t* const Fs = smem + (kt & 1) * SM::STAGE + 2 * TILE;
            if (wave < F_LOADS) {
                const int c = (wave * 32 + (lane >> 1)) ^ (((lane >> 4) & 1) << 2), h = lane & 1;
                const bool ok = c0 + c < C && 8 * h < r;
                g2lds16<TRANS>(rsF, Fs + wave * 1024, ok ? (uint32_t)((c0 + c) * r + 8 * h) * 2u : kOOB);
            }
        }
    };

    // ------------------------------------------------------------ fragment reads
    // row layout: row x of a 16-row block has x % 8 == l16 % 8, so the chunk
    // (kk * 4 + g4) ^ (l16 % 8) is a per-lane constant for each kk
    const int kc_lane = l16 * 128;
    auto chunk_of = [&](int kk) { return (((kk * 4 + g4) ^ (l16 & 7)) << 4) + kc_lane; };
    auto read_r = [&](const uint8_t* Ls, int kk, int i) -> bf16x8 {
        const uint8_t* const Rs = Ls + TILE;
        if constexpr (RQC) {
            return lds_b128(Rs + (wq * QB + i) * 2048 + chunk_of(kk));
        } else {
            const int rlo = kk * 32 + g4 * 8 + (l16 >> 2);            // rhi = rlo + 4: same swizzle
            const uint8_t* const p = Rs + rlo * 512 + (l16 & 3) * 8 + (((wq * QB + i) ^ sw512(rlo)) << 5);
            return cat_tr(lds_tr4(p), lds_tr4(p + 4 * 512));
        }
    };
    auto read_l = [&](const uint8_t* Ls, int kk, int i) -> bf16x8 {
        return lds_b128(Ls + wp * 16384 + ((i + ZROT * wq) & 7) * 2048 + chunk_of(kk));
    };
    auto read_f = [&](const uint8_t* Ls, int kk, int jt) -> bf16x8 {
        if constexpr (!TRANS) {
            return lds_b128(Ls + 2 * TILE + jt * 2048 + chunk_of(kk));
        } else {
            const int rlo = kk * 32 + g4 * 8 + (l16 >> 2);            // as read_r, 32-byte rows
            const int sw = (g4 & 1) << 2;                              // (rlo / 8) % 2 == g4 % 2
            const uint8_t* const f = Ls + 2 * TILE + (l16 & 3) * 8;
            return cat_tr(lds_tr4(f + (rlo ^ sw) * 32), lds_tr4(f + ((rlo + 4) ^ sw) * 32));
        }
    };

    f32x4 acc[QB][8];
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 zacc[JT][ZB];
#pragma unroll
    for (int i = 0; i < JT; ++i)
#pragma unroll
        for (int z = 0; z < ZB; ++z) zacc[i][z] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One 32-wide step: `pre` (the next stage's DMA, or nothing), the LDS
    // reads of the next step's fragments, and the MFMAs of `cur`.  The
    // scheduling groups at the end place one DMA after each of the first MFMAs
    // and then one fragment read after every RA MFMAs, so that neither the
    // LDS queue nor the MFMA pipe runs dry and the last read is issued well
    // before the next step needs it.
    constexpr int NR_STEP = (RQC ? QB : 2 * QB) + 8 + (ZIN ? 0 : (TRANS ? 2 * JT : JT));
    constexpr int NM_STEP = 8 * QB + (ZIN ? 0 : ZB * JT);
    auto step = [&](const Frags<JT, QB>& cur, Frags<JT, QB>& nxt, const uint8_t* nstage, int nkk, auto do_read,
                    auto pre, auto mid) {
        constexpr bool RD = decltype(do_read)::value;
        auto reads = [&] {
            if constexpr (RD) {
#pragma unroll
                for (int i = 0; i < QB; ++i) nxt.r[i] = read_r(nstage, nkk, i);
#pragma unroll
                for (int i = 0; i < 8; ++i) nxt.l[i] = read_l(nstage, nkk, i);
                if constexpr (!ZIN) {
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) nxt.f[jt] = read_f(nstage, nkk, jt);
                }
            }
        };
        auto mfmas = [&] {
#pragma unroll
            for (int pi = 0; pi < 8; ++pi)
#pragma unroll
                for (int qi = 0; qi < QB; ++qi) acc[qi][pi] = mfma16(cur.r[qi], cur.l[pi], acc[qi][pi]);
            if constexpr (!ZIN) {
#pragma unroll
                for (int jt = 0; jt < JT; ++jt)
#pragma unroll
                    for (int z = 0; z < ZB; ++z) zacc[jt][z] = mfma16(cur.f[jt], cur.l[z], zacc[jt][z]);
            }
        };
        pre();
        if constexpr (Q4) {
            // the code registers leave no room for both fragment sets during
            // the MFMAs: the reads follow them and the hardware's in-order
            // issue with the second wave of the SIMD covers their latency.
            // `mid` (the next stage's decode) is interleaved with the MFMAs:
            // its codebook reads, products and packs issue while the MFMA
            // pipe works, instead of between the steps with the pipe idle
            mfmas();
            if constexpr (std::decay_t<decltype(mid)>::active()) {
                mid();
                // the codebook reads go out over the first half of the MFMAs,
                // ahead of the products and packs that consume them
#pragma unroll
                for (int i = 0; i < NM_STEP / 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // DS read (codebook)
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);    // VALU (addresses)
                }
#pragma unroll
                for (int i = 0; i < NM_STEP / 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);    // VALU (products, packs)
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            reads();
            return;
        }
        reads();
        mfmas();
        constexpr int NV = std::decay_t<decltype(pre)>::count();
        constexpr int NR = RD ? NR_STEP : 0;
        constexpr int RA_FIT = (NM_STEP - NV) / (NR == 0 ? 1 : NR);
        constexpr int RA = RA_FIT > 2 ? RA_FIT : 2;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read (global -> LDS)
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, RA - 1, 0);
        }
    };
    struct NoPre {
        static constexpr int count() { return 0; }
        __device__ void operator()() const {}
    };
    struct StagePre {
        static constexpr int count() { return 2 * LPW; }
        decltype(issue_lr)* f;
        int kt;
        bool on;
        __device__ void operator()() const { (*f)(kt, on); }
    };
    struct NoMid {
        static constexpr bool active() { return false; }
        __device__ void operator()() const {}
    };
    struct DecodeMid {
        static constexpr bool active() { return true; }
        decltype(decode_q)* f;
        int kt;
        __device__ void operator()() const { (*f)(kt); }
    };
    using Read = std::true_type;
    using NoRead = std::false_type;

    // ------------------------------------------------------------ main loop
    const int nk = (SPLIT && slice >= 0) ? min((C + BK - 1) / BK - kbase, a.kc) : (C + BK - 1) / BK;
    if constexpr (Q4) {
        lds_barrier();                       // codebook in LDS
        issue_lr(0, true);
        issue_f(0);
        decode_q(0);
        if (nk > 1) { issue_lr(1, true); issue_f(1); }
        vmcnt_le<0>();
    } else {
        issue_lr(0, true);
        issue_f(0);
        if (nk > 1) {
            issue_lr(1, true);
            issue_f(1);
            // stage 0 landed: newer than it are stage 1's L and R loads, plus its
            // F (one load into LDS for waves 0 .. F_LOADS - 1)
            if (wave < F_LOADS) vmcnt_le<2 * LPW + 1>();
            else vmcnt_le<2 * LPW>();
        } else {
            vmcnt_le<0>();
        }
    }
    lds_barrier();

    Frags<JT, QB> fa, fb;
#pragma unroll
    for (int i = 0; i < QB; ++i) fa.r[i] = read_r(smem, 0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) fa.l[i] = read_l(smem, 0, i);
    if constexpr (!ZIN) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) fa.f[jt] = read_f(smem, 0, jt);
    }
    for (int kt = 0; kt + 1 < nk; ++kt) {
        const uint8_t* const cur = smem + (kt & 1) * SM::STAGE;
        const uint8_t* const nxt = smem + ((kt + 1) & 1) * SM::STAGE;
        // (4-bit: the R tile of stage kt + 1 decoded from the registers loaded at
        // its issue, interleaved with this step's MFMAs)
        if constexpr (Q4) step(fa, fb, cur, 1, Read{}, NoPre{}, DecodeMid{&decode_q, kt + 1});
        else step(fa, fb, cur, 1, Read{}, NoPre{}, NoMid{});
        vmcnt_le<0>();           // this wave's loads of stage kt + 1 have landed
        lds_barrier();           // ... and everyone's; stage kt's slot is free
        if constexpr (Q4) {
            if (kt + 2 < nk) { issue_lr(kt + 2, true); issue_f(kt + 2); }
            step(fb, fa, nxt, 0, Read{}, NoPre{}, NoMid{});
        } else {
            if (kt + 2 < nk) issue_f(kt + 2);
            step(fb, fa, nxt, 0, Read{}, StagePre{&issue_lr, kt + 2, kt + 2 < nk}, NoMid{});
        }
    }
    step(fa, fb, smem + ((nk - 1) & 1) * SM::STAGE, 1, Read{}, NoPre{}, NoMid{});
    step(fb, fa, smem, 0, NoRead{}, NoPre{}, NoMid{});
    vmcnt_le<0>();               // the last iteration's placeholder loads have written their zeros

    // ------------------------------------------------------------ epilogue
    // The E fragments (and Z itself when it comes precomputed) of the first 16
    // rank columns are requested before the LDS exchange so that their global
    // latency overlaps it.
    // r % 4 == 0: the four rank columns a lane needs are contiguous (16 bytes of
    // Z, 8 bytes of the forward's E = B), one load each
    const bool r4 = (r & 3) == 0;
    // fresh copies of the lane indices: the epilogue's row and column offsets
    // are then not shared with the main loop's LDS offsets, which would keep
    // them live (and spilled) across the loop
    int l16e = l16, g4e = g4;
    asm volatile("" : "+v"(l16e), "+v"(g4e));
    // E rows of output columns q in [qlo, qhi) (the member's; zeros elsewhere)
    auto load_e = [&](int jt, bf16x8 (&ef)[QB], int qlo, int qhi) {
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
            const int q = q0 + wq * QB * 16 + qi * 16 + l16e;
            const bool qok = q >= qlo && q < qhi;
            if (!TRANS && r4) {
                const int j = jt * 16 + 4 * g4e;
                u32x2 v = {0u, 0u};
                if (qok && j < r) v = *reinterpret_cast<const u32x2*>(a.E + (size_t)q * r + j);
                ef[qi] = as_bf16x8(u32x4{v[0], v[1], v[0], v[1]});
                continue;
            }
            uint32_t e4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + 4 * g4e + i;
                uint32_t v = 0u;
                if (qok && j < r) v = TRANS ? a.E[(size_t)j * Q + q] : a.E[(size_t)q * r + j];
                e4[i] = v;
            }
            const uint32_t w0 = e4[0] | (e4[1] << 16), w1 = e4[2] | (e4[3] << 16);
            ef[qi] = as_bf16x8(u32x4{w0, w1, w0, w1});
        }
    };
    // Z columns zc + j of the precomputed Z (rows of z_ld floats)
    const bool z4 = ((a.z_ld | r) & 3) == 0;
    auto load_zin = [&](int jt, f32x4 (&zv)[8], int zc) {
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int p = p0 + wp * 128 + ((pi + ZROT * wq) & 7) * 16 + l16e;
            const float* const zrow = a.Zin + (size_t)p * a.z_ld + zc;
            if (z4) {
                const int j = jt * 16 + 4 * g4e;
                zv[pi] = (p < P && j < r) ? *reinterpret_cast<const f32x4*>(zrow + j) : f32x4{0.f, 0.f, 0.f, 0.f};
                continue;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jt * 16 + 4 * g4e + i;
                zv[pi][i] = (p < P && j < r) ? zrow[j] : 0.f;
            }
        }
    };
    // member boundary i (a wave-uniform select chain: indexing the argument
    // array with a run-time value would copy the arguments to scratch memory)
    auto member_q0 = [&](int i) {
        int v = 0;
#pragma unroll
        for (int k = 0; k <= kMaxMembers; ++k) v = (k == i) ? a.member_q0[k] : v;
        return v;
    };
    // members whose output columns meet this tile (one, unless a member boundary lies inside it)
    int m_lo = 0, m_hi = 0;
    if constexpr (ZIN) {
        m_lo = kMaxMembers;
#pragma unroll
        for (int i = 0; i < kMaxMembers; ++i) {
            if (i < a.n_members && a.member_q0[i] < q0 + BQ && a.member_q0[i + 1] > q0) {
                m_lo = min(m_lo, i);
                m_hi = i;
            }
        }
    }
    // (one rank block only: with several, the prefetched block stays live
    // next to the loop-carried values and the main loop spills)
    constexpr bool PREF = RPAD == 16;
    bf16x8 ef0[QB];
    f32x4 zin0[ZIN ? 8 : 1];
    if constexpr (PREF) {
        load_e(0, ef0, ZIN ? member_q0(m_lo) : 0, ZIN ? member_q0(m_lo + 1) : Q);
        if constexpr (ZIN) load_zin(0, zin0, m_lo * r);
    }

    lds_barrier();   // every wave is done with the last stage before LDS is reused
    float* const Zx = reinterpret_cast<float*>(smem);   // [256][RPAD] float32
    // Side outputs of the rank-r product (saved U, the input gradient's V^T and
    // U^T planes): every tile of a row panel holds the panel's Z, so the panel's
    // tiles share the rows, tile qt taking rows [zr0, zr0 + zn) of the 256.  (One
    // q tile writing them all made its workgroups the last to finish: with a
    // single round of tiles they set the kernel's end.)
    const int zrows = (BP + nQt - 1) / nQt;
    const int zr0 = min(BP, qt * zrows), zn = min(BP, zr0 + zrows) - zr0;
    if constexpr (!ZIN) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int z = 0; z < ZB; ++z) {
                const int pl = wp * 128 + (wq * ZB + z) * 16 + l16e;
                *reinterpret_cast<f32x4*>(Zx + pl * RPAD + jt * 16 + 4 * g4e) = zacc[jt][z];
            }
        lds_barrier();
        if (a.Zsave != nullptr) {
            for (int e = tid; e < zn * r; e += NT) {
                const int pl = zr0 + e / r, j = e % r;
                if (p0 + pl < P)
                    a.Zsave[(size_t)(p0 + pl) * r + j] =
                        Zx[pl * RPAD + j] * (a.row_scale ? a.row_scale[p0 + pl] : 1.f);
            }
        }
        if constexpr (TRANS) {
            if (a.Zt_hi != nullptr) {
                // element (j, pl), pl fastest: runs of zn contiguous tokens per plane row
                // (planes token-block major, zt_index: p0 is a multiple of the 128-token block)
                for (int e = tid; e < zn * r; e += NT) {
                    const int j = e / zn, pl = zr0 + e % zn, p = p0 + pl;
                    if (p >= a.Mp) continue;
                    const float v = p < P ? Zx[pl * RPAD + j] * (a.row_scale ? a.row_scale[p] : 1.f) : 0.f;
                    const float u = p < P ? a.Uin[(size_t)p * r + j] : 0.f;
                    const __bf16 vh = (__bf16)v, uh = (__bf16)u;
                    const size_t o = zt_index(j, p, r);
                    a.Zt_hi[o] = __builtin_bit_cast(uint16_t, vh);
                    a.Zt_lo[o] = __builtin_bit_cast(uint16_t, (__bf16)(v - (float)vh));
                    a.Ut_hi[o] = __builtin_bit_cast(uint16_t, uh);
                    a.Ut_lo[o] = __builtin_bit_cast(uint16_t, (__bf16)(u - (float)uh));
                }
            }
        }
    }

    // precomputed Z saved row-scaled (RMSNorm in front: Zin is the product with
    // the raw input, the saved U the one with the normalised input; forward only)
    if constexpr (ZIN && !TRANS) {
        if (a.Zsave != nullptr && slice <= 0) {
            for (int e = tid; e < zn * a.z_ld; e += NT) {
                const int pl = zr0 + e / a.z_ld, j = e % a.z_ld, p = p0 + pl;
                if (p < P)
                    a.Zsave[(size_t)p * a.z_ld + j] =
                        a.Zin[(size_t)p * a.z_ld + j] * (a.row_scale ? a.row_scale[p] : 1.f);
            }
        }
    }
    const float s = a.s;
    // rank blocks of 16: the in-tile Z has RPAD columns; a precomputed one any r
    // (up to the 192 of grouped input gradients); the rank-r term goes into slice 0 only
    const int n_jt = (SPLIT && slice > 0) ? 0 : (ZIN ? (r + 15) / 16 : RPAD / 16);
    // one flat loop over (member, rank block) pairs: a nested loop here keeps
    // the accumulators live across two loop levels and spills them
    const int n_it = (m_hi - m_lo + 1) * n_jt;
    // s z as the MFMA operand: bf16 hi = bf16(s z) of 4 rank columns, then lo = bf16(s z - hi)
    auto split_hilo = [&](const f32x4& z) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float zs = z[i] * s;
            const __bf16 h = (__bf16)zs;
            hi[i] = __builtin_bit_cast(uint16_t, h);
            lo[i] = __builtin_bit_cast(uint16_t, (__bf16)(zs - (float)h));
        }
        return u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    };
    // the rank-r term of a (member, rank block) pair from fragments ef (E) and zv (Z)
    auto rank_term = [&](const bf16x8 (&ef)[QB], const f32x4 (&zv)[8]) {
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const bf16x8 zf = as_bf16x8(split_hilo(zv[pi]));
#pragma unroll
            for (int qi = 0; qi < QB; ++qi) acc[qi][pi] = mfma16(ef[qi], zf, acc[qi][pi]);
        }
    };
    if constexpr (ZIN && RPAD > 16) {
        // More than 16 precomputed rank columns: the pairs go in chunks of up to
        // ZCH whose Z and E slabs the whole workgroup first copies into LDS,
        // every load of the chunk in flight at once, then reads as fragments:
        // one global latency per chunk instead of one per rank block.  Z is
        // staged as the MFMA operand itself (s Z split into bf16 hi / lo once
        // per element, not once per wave that reads it: the split was most of
        // a rank block's cost).
        constexpr int ZCH = 4;
        constexpr int ZROW = 20;                 // 4-byte words per staged Z row (16 + 4: conflict-free 16-byte reads)
        constexpr int EROW = 24;                 // bf16 per staged E row (16 + 8)
        constexpr int ZBLK = BP * ZROW * 4, EBLK = BQ * EROW * 2;
        static_assert(ZCH * (ZBLK + EBLK) <= SM::TOTAL, "staged rank blocks fit in LDS");
        static_assert(NT == 2 * BP && NT == 2 * BQ, "staging: two threads per Z and E row");
        uint8_t* const Zst = smem;
        uint8_t* const Est = smem + ZCH * ZBLK;
        const bool e8 = (r & 7) == 0;            // forward E = B rows of r bf16: 16-byte pieces
        for (int it0 = 0; it0 < n_it; it0 += ZCH) {
            const int nb = min(ZCH, n_it - it0);
            f32x4 zl[ZCH][2];
            u32x4 el[ZCH];
#pragma unroll
            for (int b = 0; b < ZCH; ++b) {      // issue every load of the chunk
                const int it = it0 + b;
                const int mi = m_lo + it / n_jt, jt = it - (mi - m_lo) * n_jt;
                const int qlo = member_q0(mi), qhi = member_q0(mi + 1), zc = mi * r;
                const bool on = b < nb;
                {   // Z: row tid / 2, 4-float pieces 2 (tid & 1), 2 (tid & 1) + 1
                    const int p = p0 + (tid >> 1);
                    const float* const zrow = a.Zin + (size_t)p * a.z_ld + zc;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int j = jt * 16 + (2 * (tid & 1) + h) * 4;
                        f32x4 v = {0.f, 0.f, 0.f, 0.f};
                        if (on && p < P) {
                            if (z4) {
                                if (j < r) v = *reinterpret_cast<const f32x4*>(zrow + j);
                            } else {
#pragma unroll
                                for (int i = 0; i < 4; ++i) v[i] = j + i < r ? zrow[j + i] : 0.f;
                            }
                        }
                        zl[b][h] = v;
                    }
                }
                u32x4 v = {0u, 0u, 0u, 0u};
                if constexpr (!TRANS) {          // E = B: row q = q0 + tid / 2, rank columns 8 (tid & 1) ..
                    const int q = q0 + (tid >> 1), j = jt * 16 + 8 * (tid & 1);
                    if (on && q >= qlo && q < qhi && q < Q) {
                        const uint16_t* const erow = a.E + (size_t)q * r;
                        if (e8) {
                            if (j < r) v = *reinterpret_cast<const u32x4*>(erow + j);
                        } else {
                            uint32_t w[8];
#pragma unroll
                            for (int i = 0; i < 8; ++i) w[i] = j + i < r ? erow[j + i] : 0u;
                            v = u32x4{w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                                      w[6] | (w[7] << 16)};
                        }
                    }
                } else {                         // E = A: row j = jt * 16 + tid % 16, columns q0 + 8 (tid / 16) ..
                    const int j = jt * 16 + (tid & 15), q = q0 + 8 * (tid >> 4);
                    if (on && j < r && q < Q) v = *reinterpret_cast<const u32x4*>(a.E + (size_t)j * Q + q);
                }
                el[b] = v;
            }
            lds_barrier();                       // the previous chunk's fragment reads are done
#pragma unroll
            for (int b = 0; b < ZCH; ++b) {
                if (b >= nb) break;
                // row tid / 2, operand pieces g = 2 (tid & 1), 2 (tid & 1) + 1 (16 bytes each)
                uint32_t* const zs = reinterpret_cast<uint32_t*>(Zst + b * ZBLK) + (tid >> 1) * ZROW + 8 * (tid & 1);
                *reinterpret_cast<u32x4*>(zs) = split_hilo(zl[b][0]);
                *reinterpret_cast<u32x4*>(zs + 4) = split_hilo(zl[b][1]);
                uint16_t* const es = reinterpret_cast<uint16_t*>(Est + b * EBLK);
                if constexpr (!TRANS) {          // [q][j] as loaded
                    *reinterpret_cast<u32x4*>(es + (tid >> 1) * EROW + 8 * (tid & 1)) = el[b];
                } else {                         // transposed into [q][j]
                    const int jl = tid & 15, ql = 8 * (tid >> 4);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        es[(ql + i) * EROW + jl] = (uint16_t)(el[b][i >> 1] >> (16 * (i & 1)));
                }
            }
            lds_barrier();
#pragma unroll 1
            for (int b = 0; b < nb; ++b) {
                const uint16_t* const es = reinterpret_cast<const uint16_t*>(Est + b * EBLK);
                const uint32_t* const zs = reinterpret_cast<const uint32_t*>(Zst + b * ZBLK);
                bf16x8 ef[QB];
#pragma unroll
                for (int qi = 0; qi < QB; ++qi) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(es + (wq * QB * 16 + qi * 16 + l16e) * EROW + 4 * g4e);
                    ef[qi] = as_bf16x8(u32x4{v[0], v[1], v[0], v[1]});
                }
#pragma unroll
                for (int pi = 0; pi < 8; ++pi) {
                    const bf16x8 zf = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        zs + (wp * 128 + ((pi + ZROT * wq) & 7) * 16 + l16e) * ZROW + 4 * g4e));
#pragma unroll
                    for (int qi = 0; qi < QB; ++qi) acc[qi][pi] = mfma16(ef[qi], zf, acc[qi][pi]);
                }
            }
        }
    }
#pragma unroll 1
    for (int it = 0; it < ((ZIN && RPAD > 16) ? 0 : n_it); ++it) {
        const int mi = m_lo + it / max(n_jt, 1), jt = it - (mi - m_lo) * n_jt;
        const int qlo = ZIN ? member_q0(mi) : 0, qhi = ZIN ? member_q0(mi + 1) : Q, zc = mi * r;
        bf16x8 ef[QB];
        f32x4 zv[8];
        if (PREF && jt == 0 && mi == m_lo) {
#pragma unroll
            for (int qi = 0; qi < QB; ++qi) ef[qi] = ef0[qi];
            if constexpr (ZIN) {
#pragma unroll
                for (int pi = 0; pi < 8; ++pi) zv[pi] = zin0[pi];
            }
        } else {
            load_e(jt, ef, qlo, qhi);
            if constexpr (ZIN) load_zin(jt, zv, zc);
        }
        if constexpr (!ZIN) {
#pragma unroll
            for (int pi = 0; pi < 8; ++pi) {
                const int pl = wp * 128 + ((pi + ZROT * wq) & 7) * 16 + l16e;
                zv[pi] = *reinterpret_cast<const f32x4*>(Zx + pl * RPAD + jt * 16 + 4 * g4e);
            }
        }
        rank_term(ef, zv);
    }

    if (!TRANS && a.row_scale != nullptr && !(SPLIT && slice >= 0)) {   // split tiles: in split_finish
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int p = p0 + wp * 128 + ((pi + ZROT * wq) & 7) * 16 + l16e;
            const float rsc = p < P ? a.row_scale[p] : 0.f;
#pragma unroll
            for (int qi = 0; qi < QB; ++qi) acc[qi][pi] *= rsc;
        }
    }

    if (SPLIT && slice >= 0) {
        // float32 partial tile, straight from the accumulators: [slice][stile][pl][ql .. ql+3]
        const int n_stiles = nPt * nQt - a.first_split;
        float* const out = a.Part + ((size_t)slice * n_stiles + stile) * (BP * BQ);
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
            const int ql = wq * QB * 16 + qi * 16 + 4 * g4e;
#pragma unroll
            for (int pi = 0; pi < 8; ++pi) {
                const int pl = wp * 128 + ((pi + ZROT * wq) & 7) * 16 + l16e;
                *reinterpret_cast<f32x4*>(out + pl * BQ + ql) = acc[qi][pi];
            }
        }
        return;
    }

    // store: the bf16 tile goes through LDS ([256 p][256 q], 16-byte chunk c of
    // row p at c ^ (p % 32)) so that global stores are whole 512-byte row
    // segments, 16 bytes per lane.  A lane holds Out[p][q .. q+3] of each
    // accumulator (p = column l16e, q = 4 consecutive rows).
    static_assert(BP * BQ * 2 <= SM::TOTAL, "output tile must fit in LDS");
    lds_barrier();                       // Zx reads are done
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
        const int ql = wq * QB * 16 + qi * 16 + 4 * g4e;
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            const int pl = wp * 128 + ((pi + ZROT * wq) & 7) * 16 + l16e;
            const f32x4 v = acc[qi][pi];
            const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(smem + pl * 512 + (((ql >> 3) ^ (pl & 31)) << 4) + (ql & 7) * 2) = o;
        }
    }
    lds_barrier();
    const int sc = tid & 31;             // 16-byte chunk of the row
#pragma unroll 4
    for (int pass = 0; pass < BP / (NT / 32); ++pass) {
        const int pl = pass * (NT / 32) + (tid >> 5);
        const int p = p0 + pl, q = q0 + sc * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + pl * 512 + ((sc ^ (pl & 31)) << 4));
        if (p < P && q < Q) *reinterpret_cast<u32x4*>(a.Out + (size_t)p * Q + q) = v;
    }
}

// Split tiles: Out[p][q] = bf16(sum over slices k < split of Part[k][stile][pl][ql]),
// added in increasing k; each thread finishes 4 consecutive q of one tile row.
struct SplitFinishArgs {
    const float* part;
    uint16_t* out;
    int P, Q, nPt, nQt, first_split, n_stiles, split;
    const float* row_scale;     // optional per-row scale of the sum (see GemmArgs)
};

__global__ __launch_bounds__(256) void split_finish(const SplitFinishArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;        // one per 4 outputs
    if (e >= (int64_t)a.n_stiles * (g2::BP * g2::BQ / 4)) return;
    const int stile = (int)(e / (g2::BP * g2::BQ / 4));
    const int w = (int)(e % (g2::BP * g2::BQ / 4));
    const int pl = w / (g2::BQ / 4), ql = (w % (g2::BQ / 4)) * 4;
    int pt, qt;
    grouped_tile<4>(a.first_split + stile, a.nPt, a.nQt, pt, qt);
    const int p = pt * g2::BP + pl, q = qt * g2::BQ + ql;
    if (p >= a.P || q >= a.Q) return;                                 // Q % 8 == 0: q .. q+3 all valid
    const size_t ts = (size_t)g2::BP * g2::BQ;
    const float* src = a.part + (size_t)stile * ts + pl * g2::BQ + ql;
    f32x4 acc = *reinterpret_cast<const f32x4*>(src);
    for (int k = 1; k < a.split; ++k) acc += *reinterpret_cast<const f32x4*>(src + (size_t)k * a.n_stiles * ts);
    if (a.row_scale) acc *= a.row_scale[p];
    *reinterpret_cast<u32x2*>(a.out + (size_t)p * a.Q + q) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
}

}  // namespace lora
