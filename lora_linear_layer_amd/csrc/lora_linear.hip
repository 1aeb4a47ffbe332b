// C ABI of the fused LoRA linear layer (declarations and contracts in
// include/lora_linear.h).  Host side: argument validation (before any HIP
// call), workspace planning, kernel selection and launches on the caller's
// stream.  No allocation, no state, no synchronisation.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "lora_linear.h"

#include "lora_gemm.hpp"
#include "ranges.hpp"
#include "rank_stream.hpp"
#include "dequant4.hpp"
#include "merge.hpp"
#include "norm.hpp"
#include "transpose.hpp"
#include "f32_kernels.hpp"

using namespace lora;

static_assert(kMaxMembers == LORA_MAX_MEMBERS, "member table of the GEMM arguments");

namespace {

thread_local std::string g_last_error;

lora_status fail(lora_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lora_status fail(lora_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

lora_status ok() {
    g_last_error.clear();
    return LORA_OK;
}

// Kernel timer (lora_set_kernel_timer): asked for a start and a stop event
// before each kernel is enqueued; events it returns are attached to that
// kernel's dispatch (hipExtLaunchKernel), so they record the kernel itself
// without adding commands between the kernels.
std::atomic<lora_kernel_timer> g_timer{nullptr};
std::atomic<void*> g_timer_user{nullptr};

void kernel_events(const char* kernel, hipStream_t st, hipEvent_t* start, hipEvent_t* stop) {
    *start = *stop = nullptr;
    const lora_kernel_timer fn = g_timer.load(std::memory_order_acquire);
    if (!fn) return;
    void *a = nullptr, *b = nullptr;
    fn(g_timer_user.load(std::memory_order_relaxed), kernel, static_cast<void*>(st), &a, &b);
    *start = static_cast<hipEvent_t>(a);
    *stop = static_cast<hipEvent_t>(b);
}

// Every kernel of the library is enqueued through this: a plain launch, or,
// while a kernel timer is set, a launch with the timer's events attached.
#define LAUNCH(label, kernel, grid, block, shmem, stream, ...)                                          \
    do {                                                                                                \
        hipEvent_t ev0_, ev1_;                                                                          \
        kernel_events(label, stream, &ev0_, &ev1_);                                                     \
        if (ev0_ || ev1_)                                                                               \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev0_, ev1_, 0u, __VA_ARGS__);     \
        else                                                                                            \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                        \
    } while (0)

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxDim = int64_t(1) << 21;   // K, N bound: one 256-row tile stays under 2 GB
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int rpad_of(int64_t r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

// Contraction slices of a GEMM (precomputed-Z form).  An output with under
// 128 tiles of 256 x 256 splits every tile (about 256 workgroups).  With
// tail, an output of more than 256 tiles whose last round is at most half full
// also splits the tiles of that round, so it runs as a full round of shorter
// work instead of a round with idle CUs, which takes about 80 % of a full
// round's time (4-bit 2048 x 8192 -> 28672 forward 1040 -> 951-985 us, bf16
// 4096 x 4096 -> 14336 410 -> 396-402 us).  Every slice gets at least one
// 64-wide stage, and at least two when the contraction allows.
struct SplitPlan {
    int first = 0, split = 1, kc = 0;
    size_t part_floats = 0;          // float32 partial tiles in the workspace
};

SplitPlan gemm_split_plan(int64_t P, int64_t Q, int64_t C, bool tail = true) {
    SplitPlan sp;
    const int64_t T = cdiv(P, 256) * cdiv(Q, 256), nk = cdiv(C, 64);
    int64_t first = 0, want = 1;
    if (T < 128) {
        want = std::min<int64_t>(cdiv(256, T), nk / 2);
    } else if (tail && T > 256 && T % 256 != 0 && T % 256 <= 128) {
        first = T - T % 256;
        want = std::min<int64_t>(256 / (T % 256), nk / 2);
    }
    if (want < 2) return sp;
    sp.first = (int)first;
    sp.split = (int)cdiv(nk, cdiv(nk, want));
    sp.kc = (int)cdiv(nk, sp.split);
    sp.part_floats = (size_t)sp.split * (size_t)(T - first) * 256 * 256;
    return sp;
}

// Launch parameters the auto-tuner may change (lora_tune_linear).  Every
// choice stays within the workspace the plan sizes: the split modes use the
// contraction-split rules whose partial tiles it already holds, and the chunk
// counts are the model's divided by a power of two.
struct Tuning {
    int fwd_split = 0;      // forward GEMM: 0 the built-in rule (= 3), 1 no split,
    int bwd_split = 0;      //   2 few-tile outputs only, 3 also the last partial round (input gradient: bwd_split)
    int rank_div = 1;       // rank_stream token chunks: the model's count / rank_div
    int z_div_f = 1;        // rank_z_lds contraction chunks (forward U pass): the model's / z_div_f
    int z_div_b = 1;        // (backward V and U passes)
};

SplitPlan split_for(int mode, int64_t P, int64_t Q, int64_t C) {
    switch (mode) {
        case 1: return SplitPlan{};
        case 2: return gemm_split_plan(P, Q, C, false);
        default: return gemm_split_plan(P, Q, C, true);
    }
}

// Chunking of a streamed rank-r product (rank_stream): out_tiles 128-wide
// output tiles, n_ct 128-deep contraction tiles split into n_chunk chunks
// (one float32 partial per chunk).
struct RankSplit {
    int chunk_tiles = 1, n_chunk = 1;
};

constexpr int64_t kCUs = 256;          // compute units of an MI355X

RankSplit rank_split(int64_t out_tiles, int64_t n_ct, int64_t part_cols) {
    // Workgroups run in rounds of two per CU (rank_stream<32> fits three, but
    // counting them made its chunks shorter and the launch slower: 4096 tokens,
    // 4096 + 4096 columns, r = 32, 17.3 -> 18.9 us), so the streaming takes about
    // rounds x (contraction tiles per chunk) x (one 32 KB Y tile per slot);
    // each chunk adds a float32 partial of part_cols floats per 128 output
    // columns (the problems' rank columns summed over their tiles), written
    // here and read again by grad_final.  The chunk count with the least
    // bytes-equivalent cost wins, the fewest chunks on a tie.  Each chunk walks
    // at least two contraction tiles so that the double-buffered LDS ring has
    // something to overlap; at most 4 x 512 chunks are tried.  (Rounding the
    // chunk count up to fill 512 slots exactly left e.g. 576 workgroups: a
    // second round of 64.)
    RankSplit best;
    int64_t best_cost = INT64_MAX;
    const int64_t slots = 2 * kCUs, nmax = std::max<int64_t>(1, std::min<int64_t>(cdiv(n_ct, 2), 4 * slots));
    const int64_t tiles = std::max<int64_t>(out_tiles, 1);
    for (int64_t n = 1; n <= nmax; ++n) {
        const int64_t chunk = cdiv(n_ct, n), nc = cdiv(n_ct, chunk);
        const int64_t cost = cdiv(tiles * nc, slots) * chunk * (int64_t)(kRT * kRT * 2) * slots +
                             nc * part_cols * kRT * 8;
        if (cost < best_cost) {
            best_cost = cost;
            best.chunk_tiles = (int)chunk;
            best.n_chunk = (int)nc;
        }
    }
    return best;
}

// One layer as the bf16 path sees it: M tokens, K inputs, N output columns,
// rank r, and G members that share the input X (linears such as q, k and v,
// stored stacked: W [N][K], A [G r][K], B [N][r], H and dY [M][N]); member m
// owns output columns [n0[m], n0[m + 1]) and rank rows m r .. m r + r - 1 of A,
// U and V.  A plain layer is the one-member case.
struct Shape {
    int64_t M = 0, K = 0, N = 0, r = 0;
    int G = 1;
    int64_t n0[kMaxMembers + 1] = {};
    float alpha = 0.f;
    int32_t dtype = LORA_DTYPE_BF16;
    uint32_t flags = 0;
    bool norm = false;              // RMSNorm in front (1 / rms per row and A diag(g) in the workspace)
    int64_t rg() const { return (int64_t)G * r; }      // rank of the stacked A, U and V
    int64_t Nm(int m) const { return n0[m + 1] - n0[m]; }
};

Shape shape_of(const lora_linear_desc& d) {
    Shape s;
    s.M = d.M; s.K = d.K; s.N = d.N; s.r = d.r;
    s.G = 1;
    s.n0[0] = 0;
    s.n0[1] = d.N;
    s.alpha = d.alpha;
    s.dtype = d.dtype;
    s.flags = d.flags;
    return s;
}

constexpr int64_t kMaxZCols = 192;     // rank columns one rank_z_lds pass forms

// Contraction chunks of the Z pass (rank_z_lds): about 256 workgroups of 128
// rows, at least 256 columns (one F slice) per chunk.
int z_chunks(int64_t M, int64_t C) {
    const int64_t rows = cdiv(M, 128);
    return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(256, rows), cdiv(C, 256)));
}
// The adapter-gradient problems: dA^T over X in 64-rank-column slices of the
// stacked rank, dB over each member's dY columns in 64-column slices of r.
// Their output tiles (128 columns each) and rank columns set the chunking.
RankSplit split_g(const Shape& d) {
    int64_t tiles = 0, part_cols = 0;
    for (int64_t j0 = 0; j0 < d.rg(); j0 += 64) {
        tiles += cdiv(d.K, kRT);
        part_cols += cdiv(d.K, kRT) * std::min<int64_t>(d.rg() - j0, 64);
    }
    for (int m = 0; m < d.G; ++m)
        for (int64_t j0 = 0; j0 < d.r; j0 += 64) {
            tiles += cdiv(d.Nm(m), kRT);
            part_cols += cdiv(d.Nm(m), kRT) * std::min<int64_t>(d.r - j0, 64);
        }
    return rank_split(tiles, cdiv(d.M, kRT), part_cols);
}

// Workspace layout for one shape (offsets in bytes from ws).
struct Plan {
    size_t off_v = 0, off_u = 0, off_zp = 0, off_ga = 0, off_gb = 0, off_zt = 0, off_bt = 0, off_split = 0, total = 0;
    size_t off_inv = 0, off_ag = 0;     // RMSNorm in front: 1 / rms [M] float32, A diag(g) [r][K] bf16
    int64_t Mp = 0;         // tokens rounded up to a whole 128-token tile (side planes of the G pass)
    RankSplit g;
};

Plan make_plan(const Shape& d) {
    Plan p;
    const int64_t rg = d.rg();
    const size_t zbytes = align_up((size_t)d.M * rg * sizeof(float));
    p.off_v = 0;                                         // V [M][G r]
    p.off_u = zbytes;                                    // U [M][G r]
    size_t cur = 2 * zbytes;
    if (d.dtype == LORA_DTYPE_BF16) {
        const int zchunks = std::max(z_chunks(d.M, d.K), z_chunks(d.M, d.N));
        p.off_zp = cur;                                  // rank_z_lds chunk partials (one pass at a time)
        cur += align_up((size_t)zchunks * d.M * std::min(rg, kMaxZCols) * sizeof(float));
        p.g = split_g(d);
        p.off_ga = cur;                                  // dA partials [chunk][K][G r]
        cur += align_up((size_t)p.g.n_chunk * d.K * rg * sizeof(float));
        p.off_gb = cur;                                  // dB partials [chunk][N][r]
        cur += align_up((size_t)p.g.n_chunk * d.N * d.r * sizeof(float));
        p.Mp = cdiv(d.M, kRT) * kRT;
        p.off_zt = cur;                                  // V^T hi, V^T lo, U^T hi, U^T lo: bf16 [G r][Mp] each
        cur += 4 * align_up((size_t)rg * p.Mp * sizeof(uint16_t));
        p.off_bt = cur;                                  // B^T per member: bf16 [r][N_m], members side by side
        cur += align_up((size_t)d.r * d.N * sizeof(uint16_t));
        p.off_split = cur;                               // float32 partial tiles of a split contraction
        // sized for the built-in plans, which split a superset of the tiles any
        // tuned split mode splits
        const size_t n_split = std::max(gemm_split_plan(d.M, d.N, d.K).part_floats,
                                        gemm_split_plan(d.M, d.K, d.N).part_floats);
        cur += align_up(n_split * sizeof(float));
        if (d.norm) {
            p.off_inv = cur;
            cur += align_up((size_t)d.M * sizeof(float));
            p.off_ag = cur;
            cur += align_up((size_t)rg * d.K * sizeof(uint16_t));
        }
    }
    p.total = cur;
    return p;
}

lora_status check_desc(const lora_linear_desc* d, bool quant) {
    if (!d) return fail(LORA_ERR_INVALID_ARG, "desc is NULL");
    if (d->M <= 0 || d->K <= 0 || d->N <= 0 || d->r <= 0)
        return fail(LORA_ERR_INVALID_ARG, "M, K, N, r must be positive (got %lld, %lld, %lld, %lld)",
                    (long long)d->M, (long long)d->K, (long long)d->N, (long long)d->r);
    if (d->dtype != LORA_DTYPE_BF16 && d->dtype != LORA_DTYPE_F32)
        return fail(LORA_ERR_INVALID_ARG, "unknown dtype %d", (int)d->dtype);
    if (!std::isfinite(d->alpha)) return fail(LORA_ERR_INVALID_ARG, "alpha is not finite");
    if ((d->flags & ~(LORA_FLAG_ACCUM_GRADS | LORA_FLAG_W_TRANSPOSED)) != 0)
        return fail(LORA_ERR_INVALID_ARG, "unknown flag bits 0x%x", (unsigned)d->flags);
    if ((d->flags & LORA_FLAG_W_TRANSPOSED) && (quant || d->dtype != LORA_DTYPE_BF16))
        return fail(LORA_ERR_UNSUPPORTED, "LORA_FLAG_W_TRANSPOSED: bf16 weights only");
    if (d->r > 128) return fail(LORA_ERR_UNSUPPORTED, "r = %lld exceeds 128", (long long)d->r);
    if (d->K % 8 || d->N % 8)
        return fail(LORA_ERR_UNSUPPORTED, "K and N must be multiples of 8 (got K=%lld, N=%lld)",
                    (long long)d->K, (long long)d->N);
    if (d->K > kMaxDim || d->N > kMaxDim)
        return fail(LORA_ERR_UNSUPPORTED, "K and N must not exceed %lld (got K=%lld, N=%lld)", (long long)kMaxDim,
                    (long long)d->K, (long long)d->N);
    if (quant && d->K % 64) return fail(LORA_ERR_UNSUPPORTED, "4-bit weights need K %% 64 == 0 (K=%lld)", (long long)d->K);
    const int64_t big[] = {d->M * d->K, d->N * d->K, d->M * d->N, d->M * d->r};
    for (int64_t v : big)
        if (v > kMaxElems || v < 0) return fail(LORA_ERR_UNSUPPORTED, "a matrix has 2^31 or more elements");
    return LORA_OK;
}

// A group descriptor as a shape (after check_group).
Shape shape_of(const lora_group_desc& g) {
    Shape s;
    s.M = g.M; s.K = g.K; s.r = g.r;
    s.G = g.n_members;
    s.n0[0] = 0;
    for (int m = 0; m < g.n_members; ++m) s.n0[m + 1] = s.n0[m] + g.N[m];
    s.N = s.n0[g.n_members];
    s.alpha = g.alpha;
    s.dtype = g.dtype;
    s.flags = g.flags;
    return s;
}

lora_status check_group(const lora_group_desc* g) {
    if (!g) return fail(LORA_ERR_INVALID_ARG, "desc is NULL");
    if (g->n_members < 1 || g->n_members > LORA_MAX_MEMBERS)
        return fail(LORA_ERR_INVALID_ARG, "n_members = %d (1 .. %d)", (int)g->n_members, LORA_MAX_MEMBERS);
    if (g->M <= 0 || g->K <= 0 || g->r <= 0)
        return fail(LORA_ERR_INVALID_ARG, "M, K, r must be positive (got %lld, %lld, %lld)", (long long)g->M,
                    (long long)g->K, (long long)g->r);
    int64_t N = 0;
    for (int m = 0; m < g->n_members; ++m) {
        if (g->N[m] <= 0) return fail(LORA_ERR_INVALID_ARG, "member %d has N = %lld", m, (long long)g->N[m]);
        if (g->N[m] % 8) return fail(LORA_ERR_UNSUPPORTED, "member %d: N = %lld is not a multiple of 8", m,
                                     (long long)g->N[m]);
        N += g->N[m];
    }
    if (g->dtype != LORA_DTYPE_BF16 && g->dtype != LORA_DTYPE_F32)
        return fail(LORA_ERR_INVALID_ARG, "unknown dtype %d", (int)g->dtype);
    if (g->dtype != LORA_DTYPE_BF16) return fail(LORA_ERR_UNSUPPORTED, "grouped linears are bf16 only");
    if (!std::isfinite(g->alpha)) return fail(LORA_ERR_INVALID_ARG, "alpha is not finite");
    if ((g->flags & ~(LORA_FLAG_ACCUM_GRADS | LORA_FLAG_W_TRANSPOSED)) != 0)
        return fail(LORA_ERR_INVALID_ARG, "unknown flag bits 0x%x", (unsigned)g->flags);
    if (g->r > 128) return fail(LORA_ERR_UNSUPPORTED, "r = %lld exceeds 128", (long long)g->r);
    if (g->r * g->n_members > LORA_MAX_GROUP_RANK)
        return fail(LORA_ERR_UNSUPPORTED, "n_members x r = %lld exceeds %d", (long long)(g->r * g->n_members),
                    LORA_MAX_GROUP_RANK);
    if (g->K % 8) return fail(LORA_ERR_UNSUPPORTED, "K must be a multiple of 8 (K=%lld)", (long long)g->K);
    if (g->K > kMaxDim || N > kMaxDim)
        return fail(LORA_ERR_UNSUPPORTED, "K and the members' total N must not exceed %lld", (long long)kMaxDim);
    const int64_t big[] = {g->M * g->K, N * g->K, g->M * N, g->M * g->r * g->n_members};
    for (int64_t v : big)
        if (v > kMaxElems || v < 0) return fail(LORA_ERR_UNSUPPORTED, "a matrix has 2^31 or more elements");
    return LORA_OK;
}

lora_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> required,
                       std::initializer_list<std::pair<const void*, const char*>> optional) {
    for (auto& pr : required) {
        if (!pr.first) return fail(LORA_ERR_INVALID_ARG, "%s is NULL", pr.second);
        if (!aligned16(pr.first)) return fail(LORA_ERR_MISALIGNED, "%s is not 16-byte aligned", pr.second);
    }
    for (auto& pr : optional)
        if (pr.first && !aligned16(pr.first)) return fail(LORA_ERR_MISALIGNED, "%s is not 16-byte aligned", pr.second);
    return LORA_OK;
}

lora_status check_no_alias(std::initializer_list<std::pair<const void*, const char*>> outs,
                           std::initializer_list<std::pair<const void*, const char*>> all) {
    for (auto& o : outs) {
        if (!o.first) continue;
        for (auto& x : all) {
            if (x.first == o.first && x.second != o.second)
                return fail(LORA_ERR_INVALID_ARG, "output %s aliases %s", o.second, x.second);
        }
    }
    return LORA_OK;
}

lora_status check_ws(const Shape& d, void* ws, size_t ws_bytes) {
    const size_t need = make_plan(d).total;
    if (ws_bytes < need)
        return fail(LORA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    if (need > 0 && !ws) return fail(LORA_ERR_INVALID_ARG, "ws is NULL but %zu bytes are needed", need);
    if (ws && !aligned16(ws)) return fail(LORA_ERR_MISALIGNED, "ws is not 16-byte aligned");
    return LORA_OK;
}

lora_status check_ws(const lora_linear_desc& d, void* ws, size_t ws_bytes) { return check_ws(shape_of(d), ws, ws_bytes); }

lora_status launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return LORA_OK;
}

#define LAUNCH_CHECK(name) \
    do {                   \
        lora_status st_ = launched(name); \
        if (st_ != LORA_OK) return st_;   \
    } while (0)

// ---------------------------------------------------------------- bf16 launches
template <bool TRANS, int RPAD, bool ZIN, bool Q4, bool RT = false>
void launch_gemm_t(const GemmArgs& a, hipStream_t st) {
    const int tiles = (int)(cdiv(a.P, g2::BP) * cdiv(a.Q, g2::BQ));
    LAUNCH(TRANS ? "lora_gemm dX" : "lora_gemm forward", (lora_gemm<TRANS, RPAD, ZIN, Q4, false, RT>), dim3(tiles),
           dim3(g2w::NT), 0, st, a);
}

// In-tile rank-r product for r <= 16 with 16-bit weights: the forward forms
// U = X A^T and the input gradient V = dY B inside the GEMM (every q tile of
// a row panel forms it; the first one saves it).  Larger ranks, GEMMs that
// run with a split contraction and 4-bit weights take Z from the stand-alone
// streamed pass: next to the code registers and the dequantisation the
// in-tile product slows the 4-bit GEMM more than the separate pass costs
// (2048 x 8192 -> 28672, r = 16: 1403 us in-tile, 1226 us with the pass).
bool gemm_in_tile(bool quant, int r, const SplitPlan& sp) {
    return r <= 16 && !quant && sp.split == 1;
}

// The input gradient's in-tile form loads B [N][r] rows whole into LDS: 16-byte
// pieces that never straddle a row, so r is 8 or 16.
bool dx_in_tile(bool quant, int r, const SplitPlan& sp) {
    return gemm_in_tile(quant, r, sp) && r % 8 == 0;
}

// Precomputed-Z form, with the split contraction of gemm_split_plan into
// a.Part (workspace) plus split_finish when it applies.
template <bool TRANS, int RPAD, bool Q4, bool RT = false>
void launch_gemm_zin(GemmArgs a, const SplitPlan& sp, hipStream_t st) {
    if (sp.split > 1 && a.Part != nullptr) {
        a.first_split = sp.first;
        a.split = sp.split;
        a.kc = sp.kc;
        const int T = (int)(cdiv(a.P, g2::BP) * cdiv(a.Q, g2::BQ));
        const int units = sp.first + (T - sp.first) * sp.split;
        LAUNCH(TRANS ? "lora_gemm dX (split)" : "lora_gemm forward (split)", (lora_gemm<TRANS, RPAD, true, Q4, true, RT>),
               dim3(units), dim3(g2w::NT), 0, st, a);
        SplitFinishArgs f{a.Part, a.Out, a.P, a.Q, (int)cdiv(a.P, g2::BP), (int)cdiv(a.Q, g2::BQ), sp.first,
                          T - sp.first, sp.split, TRANS ? nullptr : a.row_scale};
        const int64_t n = (int64_t)(T - sp.first) * (g2::BP * g2::BQ / 4);
        LAUNCH("split_finish", split_finish, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, f);
        return;
    }
    launch_gemm_t<TRANS, RPAD, true, Q4, RT>(a, st);
}

template <bool TRANS, bool Q4, bool RT = false>
void launch_gemm(GemmArgs a, bool in_tile, const SplitPlan& sp, hipStream_t st) {
    if (a.n_members == 0) {              // a plain layer: one member over all output columns
        a.n_members = 1;
        a.member_q0[0] = 0;
        a.member_q0[1] = a.Q;
    }
    if (a.z_ld == 0) a.z_ld = a.r;
    if constexpr (!Q4) {
        if (in_tile) { launch_gemm_t<TRANS, 16, false, false, RT>(a, st); return; }
    }
    switch (rpad_of(a.r)) {
        case 16: launch_gemm_zin<TRANS, 16, Q4, RT>(a, sp, st); break;
        case 32: launch_gemm_zin<TRANS, 32, Q4, RT>(a, sp, st); break;
        case 64: launch_gemm_zin<TRANS, 64, Q4, RT>(a, sp, st); break;
        default: launch_gemm_zin<TRANS, 128, Q4, RT>(a, sp, st); break;
    }
}

// Z[m][z_j0 + j] = sum_c Y[m][c] F(j, c) for j < f_rows (Z float32 rows of z_ld;
// Y bf16 [M][C] with row stride ldy; F bf16 rows [f_rows][C]: A itself, or B^T
// from transpose_rank; or B's own rows [C][f_ld] when f_ld > 0), streamed over
// Y by rank_z_lds, up to 192 rank columns per pass.  The contraction is split into z_chunks chunks whose
// float32 partials partial_sum adds in a fixed order.  Several members (the
// linears of a group: their own columns of Y, their own F, their own rank
// columns of Z, f_rows <= 192) run as one launch; the group's chunks are
// shared out in proportion to the members' columns, so that their partials
// together fit where one pass of all the columns would put its own.
struct ZMember {
    const uint16_t* Y;      // first column of the member's Y
    const uint16_t* F;      // F rows [f_rows][C], or (f_ld > 0) B's rows [C][f_ld]
    int64_t C;
    int64_t z_j0;           // first column of the member's Z
    const float* row_scale;
    int64_t f_ld;           // 0, or B's row stride (a multiple of 8; the same for all members)
};

template <int JB, int SC, bool FB = false>
void launch_rank_z_t(const RankZArgs& a, dim3 grid, hipStream_t st) {
    LAUNCH("rank_z_lds", (rank_z_lds<JB, SC, FB>), grid, dim3(512), 0, st, a);
}

void launch_rank_z_members(int64_t M, int64_t ldy, const ZMember* mem, int G, int64_t f_rows, float* Z,
                           int64_t z_ld, float* zpart, hipStream_t st, int z_div = 1) {
    int64_t c_all = 0;
    for (int m = 0; m < G; ++m) c_all += mem[m].C;
    const int total = std::max(1, z_chunks(M, c_all) / std::max(z_div, 1));
    const bool fb = mem[0].f_ld > 0;                     // F from B's rows (callers keep f_rows <= 128)
    for (int64_t j0 = 0; j0 < f_rows; j0 += kMaxZCols) {
        const int rl = (int)std::min<int64_t>(f_rows - j0, kMaxZCols);
        const int jb = (int)cdiv(rl, 16);
        const int sc = jb > 8 ? 128 : 256;                // F slices of 16 jb rows must fit twice in LDS
        RankZArgs a{};
        a.ldy = (int)ldy;
        a.M = (int)M;
        a.f_j0 = (int)j0;
        a.rl = rl;
        a.f_ld = (int)mem[0].f_ld;
        PartialSumArgs ps{};
        ps.out = Z;
        ps.M = (int)M;
        ps.w = rl;
        ps.out_ld = (int)z_ld;
        size_t poff = 0;
        int max_used = 1;
        bool any_part = false;
        for (int m = 0; m < G; ++m) {
            const int64_t C = mem[m].C;
            const int n_chunk = G == 1 ? total : std::max<int>(1, (int)(total * C / c_all));
            const int chunk_c = (int)(cdiv(cdiv(C, n_chunk), sc) * sc);
            const int n_used = (int)cdiv(C, chunk_c);
            RankZMember& mb = a.mem[m];
            mb.Y = mem[m].Y;
            mb.F = mem[m].F;
            mb.C = (int)C;
            mb.chunk_c = chunk_c;
            mb.n_used = n_used;
            if (n_used > 1) {                             // compact partials [chunk][M][rl]
                mb.out = zpart + poff;
                mb.z_ld = rl;
                mb.z_j0 = 0;
                mb.chunk_stride = (size_t)M * rl;
                ps.part[m] = mb.out;
                ps.n_parts[m] = n_used;
                ps.out_j0[m] = (int)(mem[m].z_j0 + j0);
                ps.row_scale[m] = mem[m].row_scale;
                poff += (size_t)n_used * M * rl;
                any_part = true;
            } else {
                mb.out = Z;
                mb.z_ld = (int)z_ld;
                mb.z_j0 = (int)(mem[m].z_j0 + j0);
                mb.chunk_stride = 0;
                mb.row_scale = mem[m].row_scale;
                ps.n_parts[m] = 1;
            }
            max_used = std::max(max_used, n_used);
        }
        const dim3 grid((unsigned)cdiv(M, 128), (unsigned)max_used, (unsigned)G);
        if (fb) {
            switch (jb) {
                case 1: launch_rank_z_t<1, 256, true>(a, grid, st); break;
                case 2: launch_rank_z_t<2, 256, true>(a, grid, st); break;
                case 3: case 4: launch_rank_z_t<4, 256, true>(a, grid, st); break;
                default: launch_rank_z_t<8, 256, true>(a, grid, st); break;
            }
        } else switch (jb) {
            case 1: launch_rank_z_t<1, 256>(a, grid, st); break;
            case 2: launch_rank_z_t<2, 256>(a, grid, st); break;
            case 3: launch_rank_z_t<3, 256>(a, grid, st); break;
            case 4: launch_rank_z_t<4, 256>(a, grid, st); break;
            case 5: case 6: case 7: case 8: launch_rank_z_t<8, 256>(a, grid, st); break;
            default: launch_rank_z_t<12, 128>(a, grid, st); break;
        }
        if (any_part) {
            LAUNCH("partial_sum", partial_sum, dim3((unsigned)cdiv(M * rl, 1024), (unsigned)G), dim3(256), 0, st,
                   ps);
        }
    }
}

void launch_rank_z(int64_t M, const uint16_t* Y, int64_t ldy, int64_t C, const uint16_t* F, int64_t f_rows,
                   float* Z, int64_t z_ld, int64_t z_j0, float* zpart, hipStream_t st, int z_div = 1,
                   const float* row_scale = nullptr) {
    const ZMember one{Y, F, C, z_j0, row_scale, 0};
    launch_rank_z_members(M, ldy, &one, 1, f_rows, Z, z_ld, zpart, st, z_div);
}

// bf16 planes [G r][Mp] of V^T and U^T in the workspace: V^T hi, V^T lo, U^T hi, U^T lo.
uint16_t* zt_plane(const Plan& plan, char* wsb, int64_t rows, int i) {
    const size_t plane = align_up((size_t)rows * plan.Mp * sizeof(uint16_t));
    return reinterpret_cast<uint16_t*>(wsb + plan.off_zt + i * plane);
}

// dA and dB from X, V and dY, U: rank_stream partials (dA = s V^T X over the
// stacked rank in 64-column problems; dB = s dY_m^T U_m per member), then the
// fixed-order final sum, scale, dtype and layout.  planes_ready: the dX GEMM
// has already written the hi / lo planes of V^T and U^T (V is then not read);
// otherwise zt_hilo writes them.  Problems of one rank width share a launch.
lora_status launch_adapter_grads(const Shape& d, const Plan& plan, char* wsb, const uint16_t* X, const float* V,
                                 const uint16_t* dY, const float* U, void* dA, void* dB, bool planes_ready,
                                 hipStream_t st, int rank_div = 1, const float* v_row_scale = nullptr,
                                 const uint16_t* a_col_scale = nullptr) {
    const int64_t rg = d.rg();
    // token chunks: the model's count, or fewer (tuned); the partials fit either way
    RankSplit g = plan.g;
    if (rank_div > 1) {
        const int64_t n_ct = cdiv(d.M, kRT);
        g.chunk_tiles = (int)cdiv(n_ct, std::max<int64_t>(1, plan.g.n_chunk / rank_div));
        g.n_chunk = (int)cdiv(n_ct, g.chunk_tiles);
    }
    float* const ga = reinterpret_cast<float*>(wsb + plan.off_ga);
    float* const gb = reinterpret_cast<float*>(wsb + plan.off_gb);
    uint16_t* const vt_hi = zt_plane(plan, wsb, rg, 0);
    uint16_t* const vt_lo = zt_plane(plan, wsb, rg, 1);
    uint16_t* const ut_hi = zt_plane(plan, wsb, rg, 2);
    uint16_t* const ut_lo = zt_plane(plan, wsb, rg, 3);
    if (!planes_ready) {
        const int zt_tiled = rg >= 32 ? 1 : 0;
        const int64_t zt_blocks = zt_tiled ? (plan.Mp / kSideBlock) * cdiv(rg, 32) : cdiv(rg * plan.Mp, 256);
        LAUNCH("zt_hilo", zt_hilo, dim3((unsigned)zt_blocks, 2), dim3(256), 0, st, V, U, vt_hi, vt_lo, ut_hi,
               ut_lo, (int)d.M, (int)plan.Mp, (int)rg, v_row_scale, zt_tiled);
        LAUNCH_CHECK("zt_hilo");
    }
    // the problems, by rank padding (16, 32 or 64 columns)
    RankProblem probs[3][4 * kMaxMembers];
    int np[3] = {0, 0, 0};
    auto pad_slot = [](int64_t rl) { return rl <= 16 ? 0 : rl <= 32 ? 1 : 2; };
    for (int64_t j0 = 0; j0 < rg; j0 += 64) {            // dA^T [K][G r]: 64 rank columns per problem
        const int64_t rl = std::min<int64_t>(rg - j0, 64);
        const int sl = pad_slot(rl);
        probs[sl][np[sl]++] = RankProblem{X, vt_hi, vt_lo, ga, (int)d.K, (int)d.K, (int)cdiv(d.K, kRT),
                                          (int)rg, (int)j0, (int)rl, (int)rg, (int)j0, (size_t)d.K * rg};
    }
    for (int m = 0; m < d.G; ++m) {                       // dB [N][r]: member m's rows from its dY columns
        for (int64_t j0 = 0; j0 < d.r; j0 += 64) {
            const int64_t rl = std::min<int64_t>(d.r - j0, 64);
            const int sl = pad_slot(rl);
            probs[sl][np[sl]++] = RankProblem{dY + d.n0[m], ut_hi, ut_lo, gb + (size_t)d.n0[m] * d.r, (int)d.Nm(m),
                                              (int)d.N, (int)cdiv(d.Nm(m), kRT), (int)rg, (int)(m * d.r + j0),
                                              (int)rl, (int)d.r, (int)j0, (size_t)d.N * d.r};
        }
    }
    for (int sl = 0; sl < 3; ++sl) {
        for (int p0 = 0; p0 < np[sl]; p0 += kMaxRankProblems) {
            RankArgs a{};
            a.n_prob = std::min(np[sl] - p0, kMaxRankProblems);
            int tiles = 1;
            for (int i = 0; i < a.n_prob; ++i) {
                a.prob[i] = probs[sl][p0 + i];
                tiles = std::max(tiles, a.prob[i].n_tiles);
            }
            a.M = (int)d.M;
            a.chunk_tiles = g.chunk_tiles;
            a.n_chunk = g.n_chunk;
            const dim3 grid((unsigned)tiles, (unsigned)a.n_chunk, (unsigned)a.n_prob);
            switch (sl) {
                case 0: LAUNCH("rank_stream", (rank_stream<16>), grid, dim3(256), 0, st, a); break;
                case 1: LAUNCH("rank_stream", (rank_stream<32>), grid, dim3(256), 0, st, a); break;
                default: LAUNCH("rank_stream", (rank_stream<64>), grid, dim3(256), 0, st, a); break;
            }
        }
    }
    LAUNCH_CHECK("rank_stream(dA, dB)");
    GradFinalArgs f{};
    f.ga = ga;
    f.gb = gb;
    f.dA = dA;
    f.dB = dB;
    f.K = (int)d.K;
    f.N = (int)d.N;
    f.ra = (int)rg;
    f.rb = (int)d.r;
    f.n_chunk = g.n_chunk;
    f.s = d.alpha / (float)d.r;
    f.f32_out = 0;
    f.accumulate = (d.flags & LORA_FLAG_ACCUM_GRADS) ? 1 : 0;
    f.a_col_scale = a_col_scale;
    f.tiled = rg >= 64 ? 1 : 0;
    const int64_t n_tiles = f.tiled ? cdiv(d.K, 64) * cdiv(rg, 64) : 0;
    const int64_t n_flat = (f.tiled ? 0 : d.K * rg) + d.N * d.r;
    LAUNCH("grad_final", grad_final, dim3((unsigned)(n_tiles + cdiv(n_flat, 256))), dim3(256), 0, st, f);
    LAUNCH_CHECK("grad_final");
    return LORA_OK;
}

// member boundaries of the forward GEMM's epilogue
void set_members(GemmArgs& g, const Shape& d) {
    g.n_members = d.G;
    for (int m = 0; m <= d.G; ++m) g.member_q0[m] = (int)d.n0[m];
}

// ---------------------------------------------------------------- forward
lora_status fwd_bf16(const Shape& d, bool quant, const void* X, const void* W, const uint8_t* Wq,
                     const uint16_t* absmax, const float* codebook, const void* A, const void* B, void* H,
                     float* U_save, void* ws, hipStream_t st, const Tuning& tn = Tuning{},
                     const float* row_scale = nullptr) {
    const Plan plan = make_plan(d);
    char* const wsb = static_cast<char*>(ws);
    const int r = (int)d.r;
    const uint16_t* const X16 = static_cast<const uint16_t*>(X);
    const uint16_t* const A16 = static_cast<const uint16_t*>(A);
    float* const zpart = reinterpret_cast<float*>(wsb + plan.off_zp);
    const SplitPlan sp = split_for(tn.fwd_split, d.M, d.N, d.K);
    const bool in_tile = d.G == 1 && gemm_in_tile(quant, r, sp);
    float* U = U_save;
    if (!in_tile) {
        // U = X A^T (all members in one pass over X), read by the GEMM epilogue; with
        // a row scale the pass forms the raw product and the GEMM saves it scaled
        if (!U || row_scale) U = reinterpret_cast<float*>(wsb + plan.off_u);
        launch_rank_z(d.M, X16, d.K, d.K, A16, d.rg(), U, d.rg(), 0, zpart, st, tn.z_div_f);
        LAUNCH_CHECK("rank_z_lds(U)");
    }
    GemmArgs g{};
    g.L = X16;
    g.R = static_cast<const uint16_t*>(W);
    g.Rq = Wq;
    g.Rabs = absmax;
    g.codebook = codebook;
    g.F = A16;
    g.E = static_cast<const uint16_t*>(B);
    g.Out = static_cast<uint16_t*>(H);
    g.Zsave = (in_tile || row_scale) ? U_save : nullptr;
    g.Zin = in_tile ? nullptr : U;
    g.z_ld = (int)d.rg();
    g.row_scale = row_scale;
    set_members(g, d);
    g.Part = reinterpret_cast<float*>(wsb + plan.off_split);
    g.P = (int)d.M; g.Q = (int)d.N; g.C = (int)d.K; g.r = r;
    g.s = d.alpha / (float)d.r;
    if (quant) launch_gemm<false, true>(g, in_tile, sp, st);
    else launch_gemm<false, false>(g, in_tile, sp, st);
    LAUNCH_CHECK(quant ? "lora_gemm(4-bit forward)" : "lora_gemm(forward)");
    return ok();
}

// ---------------------------------------------------------------- backward
// Order on the stream: U (if not saved) -> dX GEMM, which forms V = dY B in
// the tile for a plain layer with r = 8 or 16 (16-bit W) and saves it, or takes
// V from streamed passes (one per member, over the member's dY columns) ->
// dA, dB partials -> final sum.  With several members the dX GEMM contracts
// over all their output columns at once: dX = sum_m (dY_m W_m + s V_m A_m).
lora_status bwd_bf16(const Shape& d, bool quant, const void* dY, const void* X, const void* W,
                     const uint8_t* Wq, const uint16_t* absmax, const float* codebook, const void* A,
                     const void* B, const float* U_saved, void* dX, void* dA, void* dB, void* ws, hipStream_t st,
                     const Tuning& tn = Tuning{}, const float* row_scale = nullptr,
                     const uint16_t* a_col_scale = nullptr) {
    const Plan plan = make_plan(d);
    const int r = (int)d.r;
    const int64_t rg = d.rg();
    char* const wsb = static_cast<char*>(ws);
    float* const V = reinterpret_cast<float*>(wsb + plan.off_v);
    float* const zpart = reinterpret_cast<float*>(wsb + plan.off_zp);
    const uint16_t* const dY16 = static_cast<const uint16_t*>(dY);
    const uint16_t* const X16 = static_cast<const uint16_t*>(X);
    const uint16_t* const A16 = static_cast<const uint16_t*>(A);
    const uint16_t* const B16 = static_cast<const uint16_t*>(B);

    // 1. U (saved by the forward, or rebuilt from X)
    const float* U = U_saved;
    if (!U) {
        float* Uw = reinterpret_cast<float*>(wsb + plan.off_u);
        launch_rank_z(d.M, X16, d.K, d.K, A16, rg, Uw, rg, 0, zpart, st, tn.z_div_b, row_scale);
        LAUNCH_CHECK("rank_z_lds(U)");
        U = Uw;
    }
    // 2. V = dY B: inside the dX GEMM when it runs in the in-tile form,
    //    else the streamed pass of each member over its columns of dY
    const SplitPlan sp = split_for(tn.bwd_split, d.M, d.K, d.N);
    const bool v_in_tile = dX != nullptr && d.G == 1 && dx_in_tile(quant, r, sp);
    if (!v_in_tile) {
        // B's rows are whole 16-byte pieces when r % 8 == 0: the pass reads B
        // itself (its slices hold up to 128 rank columns, r's limit); otherwise
        // transpose_rank writes every member's B^T first
        const bool b_rows = d.r % 8 == 0 && d.r <= 128;
        uint16_t* const BT = reinterpret_cast<uint16_t*>(wsb + plan.off_bt);
        if (!b_rows) {
            TransposeRankArgs ta{};
            ta.G = d.G;
            ta.r = r;
            for (int m = 0; m <= d.G; ++m) ta.n0[m] = (int)d.n0[m];
            LAUNCH("transpose_rank", transpose_rank, dim3((unsigned)cdiv(d.r * d.N, 256)), dim3(256), 0, st, B16,
                   BT, ta);
        }
        ZMember mem[kMaxMembers];
        for (int m = 0; m < d.G; ++m)
            mem[m] = b_rows ? ZMember{dY16 + d.n0[m], B16 + (size_t)d.n0[m] * d.r, d.Nm(m), (int64_t)m * d.r,
                                      nullptr, d.r}
                            : ZMember{dY16 + d.n0[m], BT + (size_t)d.r * d.n0[m], d.Nm(m), (int64_t)m * d.r,
                                      nullptr, 0};
        launch_rank_z_members(d.M, d.N, mem, d.G, d.r, V, rg, zpart, st, tn.z_div_b);
        LAUNCH_CHECK("rank_z_lds(V)");
    }
    // 3. dX = dY W + s V A  (summed over the members: one contraction over all N columns)
    if (dX) {
        GemmArgs g{};
        g.L = dY16;
        g.R = static_cast<const uint16_t*>(W);
        g.Rq = Wq;
        g.Rabs = absmax;
        g.codebook = codebook;
        g.F = B16;
        g.E = A16;
        g.Out = static_cast<uint16_t*>(dX);
        g.Zin = v_in_tile ? nullptr : V;
        g.z_ld = (int)rg;
        if (v_in_tile) {
            // V goes straight into the adapter-gradient planes (with U's), not to V [M][r]
            g.Zt_hi = zt_plane(plan, wsb, rg, 0);
            g.Zt_lo = zt_plane(plan, wsb, rg, 1);
            g.Ut_hi = zt_plane(plan, wsb, rg, 2);
            g.Ut_lo = zt_plane(plan, wsb, rg, 3);
            g.Uin = U;
            g.Mp = (int)plan.Mp;
        }
        g.Part = reinterpret_cast<float*>(wsb + plan.off_split);
        g.row_scale = row_scale;
        g.P = (int)d.M; g.Q = (int)d.K; g.C = (int)d.N; g.r = (int)rg;
        g.s = d.alpha / (float)d.r;
        if (quant) launch_gemm<true, true>(g, v_in_tile, sp, st);
        else if (d.flags & LORA_FLAG_W_TRANSPOSED) launch_gemm<true, false, true>(g, v_in_tile, sp, st);
        else launch_gemm<true, false>(g, v_in_tile, sp, st);
        LAUNCH_CHECK(quant ? "lora_gemm(4-bit dX)" : "lora_gemm(dX)");
    }
    // 4., 5. dA = s V^T X, dB = s dY^T U
    const lora_status gst = launch_adapter_grads(d, plan, wsb, X16, V, dY16, U, dA, dB, v_in_tile, st, tn.rank_div,
                                                 row_scale, a_col_scale);
    if (gst != LORA_OK) return gst;
    return ok();
}

// ---------------------------------------------------------------- float32 mode
template <int RMODE>
void launch_f32_fused(const F32FusedArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)cdiv(a.Q, 64), (unsigned)cdiv(a.P, 64));
    LAUNCH("f32_fused", (f32_fused<RMODE>), grid, dim3(256), 0, st, a);
}

void launch_f32_fused_mode(int rmode, const F32FusedArgs& a, hipStream_t st) {
    switch (rmode) {
        case kRDirect: launch_f32_fused<kRDirect>(a, st); break;
        case kRTrans: launch_f32_fused<kRTrans>(a, st); break;
        case kRQuantDirect: launch_f32_fused<kRQuantDirect>(a, st); break;
        default: launch_f32_fused<kRQuantTrans>(a, st); break;
    }
}

lora_status fwd_f32(const lora_linear_desc& d, bool quant, const void* X, const void* W, const uint8_t* Wq,
                    const uint16_t* absmax, const float* codebook, const void* A, const void* B, void* H,
                    float* U_save, void* ws, hipStream_t st) {
    const Plan plan = make_plan(shape_of(d));
    float* U = U_save ? U_save : reinterpret_cast<float*>(static_cast<char*>(ws) + plan.off_u);
    const int M = (int)d.M, K = (int)d.K, N = (int)d.N, r = (int)d.r;
    LAUNCH("f32_skinny", f32_skinny, dim3((unsigned)cdiv((int64_t)M * r, 256)), dim3(256), 0, st,
                       static_cast<const float*>(X), static_cast<const float*>(A), U, M, K, r, 0);
    LAUNCH_CHECK("f32_skinny(U)");
    F32FusedArgs a{};
    a.L = static_cast<const float*>(X);
    a.R = static_cast<const float*>(W);
    a.Rq = Wq; a.Rabs = absmax; a.codebook = codebook;
    a.E = static_cast<const float*>(B);
    a.Z = U;
    a.Out = static_cast<float*>(H);
    a.P = M; a.Q = N; a.C = K; a.r = r; a.e_trans = 0;
    a.s = d.alpha / (float)d.r;
    launch_f32_fused_mode(quant ? kRQuantDirect : kRDirect, a, st);
    LAUNCH_CHECK("f32_fused(forward)");
    return ok();
}

lora_status bwd_f32(const lora_linear_desc& d, bool quant, const void* dY, const void* X, const void* W,
                    const uint8_t* Wq, const uint16_t* absmax, const float* codebook, const void* A, const void* B,
                    const float* U_saved, void* dX, void* dA, void* dB, void* ws, hipStream_t st) {
    const Plan plan = make_plan(shape_of(d));
    char* const wsb = static_cast<char*>(ws);
    float* const V = reinterpret_cast<float*>(wsb + plan.off_v);
    const int M = (int)d.M, K = (int)d.K, N = (int)d.N, r = (int)d.r;
    const float s = d.alpha / (float)d.r;
    const float* dYf = static_cast<const float*>(dY);
    const float* Xf = static_cast<const float*>(X);
    LAUNCH("f32_skinny", f32_skinny, dim3((unsigned)cdiv((int64_t)M * r, 256)), dim3(256), 0, st,
                       dYf, static_cast<const float*>(B), V, M, N, r, 1);
    LAUNCH_CHECK("f32_skinny(V)");
    const float* U = U_saved;
    if (!U) {
        float* Uw = reinterpret_cast<float*>(wsb + plan.off_u);
        LAUNCH("f32_skinny", f32_skinny, dim3((unsigned)cdiv((int64_t)M * r, 256)), dim3(256), 0, st,
                           Xf, static_cast<const float*>(A), Uw, M, K, r, 0);
        LAUNCH_CHECK("f32_skinny(U)");
        U = Uw;
    }
    if (dX) {
        F32FusedArgs a{};
        a.L = dYf;
        a.R = static_cast<const float*>(W);
        a.Rq = Wq; a.Rabs = absmax; a.codebook = codebook;
        a.E = static_cast<const float*>(A);
        a.Z = V;
        a.Out = static_cast<float*>(dX);
        a.P = M; a.Q = K; a.C = N; a.r = r; a.e_trans = 1;
        a.s = s;
        launch_f32_fused_mode(quant ? kRQuantTrans : kRTrans, a, st);
        LAUNCH_CHECK("f32_fused(dX)");
    }
    const int acc = (d.flags & LORA_FLAG_ACCUM_GRADS) ? 1 : 0;
    LAUNCH("f32_grad", f32_grad, dim3((unsigned)cdiv((int64_t)K * r, 256)), dim3(256), 0, st,
                       Xf, (const float*)V, static_cast<float*>(dA), M, K, r, s, 1, acc);
    LAUNCH_CHECK("f32_grad(dA)");
    LAUNCH("f32_grad", f32_grad, dim3((unsigned)cdiv((int64_t)N * r, 256)), dim3(256), 0, st,
                       dYf, U, static_cast<float*>(dB), M, N, r, s, 0, acc);
    LAUNCH_CHECK("f32_grad(dB)");
    return ok();
}

// ---------------------------------------------------------------- allocation-free backward
// The backward's intermediates (V, U, the rank planes, the split-M partials)
// live in this array when the caller cannot provide a workspace.  Its address
// differs on every device: the host looks it up once per device with
// hipGetSymbolAddress and never uses the name itself as an address.
constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current).
lora_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LORA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(LORA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LORA_OK;
}

// Bytes of the backward's intermediates for a 16-bit weight: the workspace
// layout up to its last region, plus the float32 slices of the input
// gradient's own split contraction (the workspace holds the larger of the
// forward's and the input gradient's).
size_t bwd_scratch_bytes(const Shape& d) {
    const Plan p = make_plan(d);
    if (d.dtype != LORA_DTYPE_BF16) return p.total;
    return p.off_split + align_up(gemm_split_plan(d.M, d.K, d.N).part_floats * sizeof(float));
}

// ---------------------------------------------------------------- auto-tuner
// Tuned launch parameters per (device, shape): chosen by lora_tune_linear from
// timed runs, kept for the process, saved to and loaded from a text file.
struct TuneKey {
    std::string arch;
    int cus;
    int64_t M, K, N, r;
    int quant;
    bool operator<(const TuneKey& o) const {
        return std::tie(arch, cus, M, K, N, r, quant) < std::tie(o.arch, o.cus, o.M, o.K, o.N, o.r, o.quant);
    }
};

std::mutex g_tune_mu;
std::map<TuneKey, Tuning> g_tuned;
std::atomic<bool> g_tune_any{false};

struct DevInfo {
    std::string arch;
    int cus = 0;
    bool ok = false;
};
DevInfo g_devinfo[kMaxDevices];
std::mutex g_dev_mu;

// Architecture name (without feature suffixes) and compute-unit count of the
// current device, looked up once per device.
bool current_device_info(std::string& arch, int& cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DevInfo& di = g_devinfo[dev];
    if (!di.ok) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        std::string a = prop.gcnArchName;
        di.arch = a.substr(0, a.find(':'));
        di.cus = prop.multiProcessorCount;
        di.ok = true;
    }
    arch = di.arch;
    cus = di.cus;
    return true;
}

TuneKey tune_key(const std::string& arch, int cus, const lora_linear_desc& d, bool quant) {
    return TuneKey{arch, cus, d.M, d.K, d.N, d.r, quant ? 1 : 0};
}

// The tuned parameters for a plain bf16 layer on the current device, or the
// built-in rules when the cache holds none (no lookup at all while it is empty).
Tuning tuned_for(const lora_linear_desc& d, bool quant) {
    if (!g_tune_any.load(std::memory_order_acquire) || d.dtype != LORA_DTYPE_BF16) return Tuning{};
    std::string arch;
    int cus = 0;
    if (!current_device_info(arch, cus)) return Tuning{};
    std::lock_guard<std::mutex> lock(g_tune_mu);
    const auto it = g_tuned.find(tune_key(arch, cus, d, quant));
    return it == g_tuned.end() ? Tuning{} : it->second;
}

bool valid_tuning(const Tuning& t) {
    auto pow2 = [](int v) { return v == 1 || v == 2 || v == 4 || v == 8; };
    return t.fwd_split >= 0 && t.fwd_split <= 3 && t.bwd_split >= 0 && t.bwd_split <= 3 && pow2(t.rank_div) &&
           pow2(t.z_div_f) && pow2(t.z_div_b);
}

// ---------------------------------------------------------------- buffer ranges
// Every buffer resource the bf16 kernels of one descriptor may build, with the
// largest range it asks for (the first workgroup and step, where the clipping
// to the matrix ends has not yet shortened it).  The kernels build their
// resources with the same functions (ranges.hpp); a call that skips dX or does
// not pass U builds a subset.
struct RangeList {
    lora_buffer_range* out;
    int cap, n;
    void add(const char* kernel, const char* operand, uint64_t bytes) {
        if (out && n < cap) out[n] = lora_buffer_range{kernel, operand, bytes};
        ++n;
    }
};

void gemm_ranges(RangeList& L, const char* name, bool trans, bool quant, bool in_tile, int64_t P, int64_t Q,
                 int64_t C, int64_t r, bool wt = false) {
    L.add(name, trans ? "dY panel" : "X panel", panel_bytes(P, 0, g2::BP, C));
    if (!quant) {
        if (trans && !wt) L.add(name, "W stage (rows c0 .. c0 + 63)", gemm_wt_stage_bytes(C, Q, 0, 0));
        else L.add(name, trans ? "W^T panel" : "W panel", panel_bytes(Q, 0, g2::BQ, C));
    } else if (!trans) {
        L.add(name, "4-bit codes (256 rows)", (uint64_t)q4_code_bytes<int64_t>(Q, 0, g2::BQ, C, 0));
        L.add(name, "absmax (256 rows)", (uint64_t)q4_absmax_bytes<int64_t>(Q, 0, g2::BQ, C, 0));
    }
    if (in_tile) L.add(name, trans ? "B" : "A", trans ? whole_bytes(C, r) : whole_bytes(r, C));
}

void rank_z_ranges(RangeList& L, const char* name, int64_t M, int64_t C, int64_t ldy, int64_t f_rows) {
    L.add(name, "Y block (128 rows)", strided_panel_bytes(M, 0, 128, C, ldy));
    L.add(name, "F rows", whole_bytes(std::min(f_rows, kMaxZCols), C));
}

void buffer_ranges(const Shape& d, bool quant, RangeList& L) {
    if (d.dtype != LORA_DTYPE_BF16) return;          // the float32 mode uses plain loads only
    const int r = (int)d.r;
    const int64_t rg = d.rg();
    const SplitPlan spf = gemm_split_plan(d.M, d.N, d.K);
    const SplitPlan spb = gemm_split_plan(d.M, d.K, d.N);
    // forward (U by the streamed pass when it is not formed in the tile)
    const bool fwd_in_tile = d.G == 1 && gemm_in_tile(quant, r, spf);
    rank_z_ranges(L, "rank_z_lds (U = X A^T)", d.M, d.K, d.K, rg);   // forward, or a backward without U
    gemm_ranges(L, "lora_gemm (forward)", false, quant, fwd_in_tile, d.M, d.N, d.K, d.r);
    // backward: V streamed per member unless the dX GEMM forms it
    for (int m = 0; m < d.G; ++m) rank_z_ranges(L, "rank_z_lds (V = dY B)", d.M, d.Nm(m), d.N, d.r);
    gemm_ranges(L, "lora_gemm (dX)", true, quant, d.G == 1 && dx_in_tile(quant, r, spb), d.M, d.K, d.N, d.r,
                (d.flags & LORA_FLAG_W_TRANSPOSED) != 0);
    for (int64_t j0 = 0; j0 < rg; j0 += 64) {
        const int64_t rl = std::min<int64_t>(rg - j0, 64);
        const int64_t TM = rpad_of(rl) <= 16 ? kRT : kRT / 2;
        L.add("rank_stream (dA partials)", "X step", stream_y_bytes(d.M, d.K, 0, 0, TM, d.K));
        L.add("rank_stream (dA partials)", "rank plane block (hi, lo)", stream_side_bytes(rl, TM));
    }
    for (int m = 0; m < d.G; ++m) {
        for (int64_t j0 = 0; j0 < d.r; j0 += 64) {
            const int64_t rl = std::min<int64_t>(d.r - j0, 64);
            const int64_t TM = rpad_of(rl) <= 16 ? kRT : kRT / 2;
            L.add("rank_stream (dB partials)", "dY step", stream_y_bytes(d.M, d.Nm(m), 0, 0, TM, d.N));
            L.add("rank_stream (dB partials)", "rank plane block (hi, lo)", stream_side_bytes(rl, TM));
        }
    }
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* lora_status_string(lora_status s) {
    switch (s) {
        case LORA_OK: return "ok";
        case LORA_ERR_INVALID_ARG: return "invalid argument";
        case LORA_ERR_UNSUPPORTED: return "unsupported shape or option";
        case LORA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case LORA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case LORA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* lora_last_error(void) { return g_last_error.c_str(); }

void lora_set_kernel_timer(lora_kernel_timer fn, void* user) {
    g_timer_user.store(user, std::memory_order_relaxed);
    g_timer.store(fn, std::memory_order_release);
}

lora_status lora_linear_workspace_size(const lora_linear_desc* desc, size_t* bytes) {
    if (!bytes) return fail(LORA_ERR_INVALID_ARG, "bytes is NULL");
    lora_status st = check_desc(desc, false);
    if (st != LORA_OK) return st;
    *bytes = make_plan(shape_of(*desc)).total;
    return ok();
}

lora_status lora_linear_buffer_ranges(const lora_linear_desc* desc, int32_t quant, lora_buffer_range* out,
                                      int32_t capacity, int32_t* count) {
    if (!count) return fail(LORA_ERR_INVALID_ARG, "count is NULL");
    if (capacity < 0 || (capacity > 0 && !out)) return fail(LORA_ERR_INVALID_ARG, "out is NULL or capacity < 0");
    lora_status st = check_desc(desc, quant != 0);
    if (st != LORA_OK) return st;
    RangeList L{out, capacity, 0};
    buffer_ranges(shape_of(*desc), quant != 0, L);
    *count = L.n;
    return ok();
}

lora_status lora_linear_bwd_noalloc(const lora_linear_desc* desc, const void* dY, const void* X, const void* W,
                                    const void* A, const void* B, const float* U_saved, void* dX, void* dA, void* dB,
                                    void* stream) {
    lora_status st = check_desc(desc, false);
    if (st != LORA_OK) return st;
    st = check_ptrs({{dY, "dY"}, {X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {dA, "dA"}, {dB, "dB"}},
                    {{U_saved, "U_saved"}, {dX, "dX"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                        {{dY, "dY"}, {X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {U_saved, "U_saved"},
                         {dX, "dX"}, {dA, "dA"}, {dB, "dB"}});
    if (st != LORA_OK) return st;
    const size_t need = bwd_scratch_bytes(shape_of(*desc));
    if (need > kScratchBytes)
        return fail(LORA_ERR_UNSUPPORTED,
                    "this backward needs %zu bytes of intermediates; the allocation-free entry point holds %zu "
                    "(use lora_linear_bwd with a workspace)", need, kScratchBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != LORA_OK) return st;
    if (s) {
        hipDevice_t sd = -1;
        int cur = -1;
        if (hipStreamGetDevice(s, &sd) == hipSuccess && hipGetDevice(&cur) == hipSuccess && sd != cur)
            return fail(LORA_ERR_INVALID_ARG, "stream belongs to device %d but device %d is current", (int)sd, cur);
    }
    if (desc->dtype == LORA_DTYPE_F32)
        return bwd_f32(*desc, false, dY, X, W, nullptr, nullptr, nullptr, A, B, U_saved, dX, dA, dB, ws, s);
    return bwd_bf16(shape_of(*desc), false, dY, X, W, nullptr, nullptr, nullptr, A, B, U_saved, dX, dA, dB, ws, s);
}

lora_status lora_group_workspace_size(const lora_group_desc* desc, size_t* bytes) {
    if (!bytes) return fail(LORA_ERR_INVALID_ARG, "bytes is NULL");
    lora_status st = check_group(desc);
    if (st != LORA_OK) return st;
    *bytes = make_plan(shape_of(*desc)).total;
    return ok();
}

lora_status lora_group_fwd(const lora_group_desc* desc, const void* X, const void* W, const void* A, const void* B,
                           void* H, float* U_save, void* ws, size_t ws_bytes, void* stream) {
    lora_status st = check_group(desc);
    if (st != LORA_OK) return st;
    st = check_ptrs({{X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {H, "H"}}, {{U_save, "U_save"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{H, "H"}, {U_save, "U_save"}},
                        {{X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {H, "H"}, {U_save, "U_save"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    const Shape d = shape_of(*desc);
    st = check_ws(d, ws, ws_bytes);
    if (st != LORA_OK) return st;
    return fwd_bf16(d, false, X, W, nullptr, nullptr, nullptr, A, B, H, U_save, ws, static_cast<hipStream_t>(stream));
}

lora_status lora_group_bwd(const lora_group_desc* desc, const void* dY, const void* X, const void* W, const void* A,
                           const void* B, const float* U_saved, void* dX, void* dA, void* dB, void* ws,
                           size_t ws_bytes, void* stream) {
    lora_status st = check_group(desc);
    if (st != LORA_OK) return st;
    st = check_ptrs({{dY, "dY"}, {X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {dA, "dA"}, {dB, "dB"}},
                    {{U_saved, "U_saved"}, {dX, "dX"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                        {{dY, "dY"}, {X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {U_saved, "U_saved"},
                         {dX, "dX"}, {dA, "dA"}, {dB, "dB"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    const Shape d = shape_of(*desc);
    st = check_ws(d, ws, ws_bytes);
    if (st != LORA_OK) return st;
    return bwd_bf16(d, false, dY, X, W, nullptr, nullptr, nullptr, A, B, U_saved, dX, dA, dB, ws,
                    static_cast<hipStream_t>(stream));
}

lora_status lora_linear_fwd(const lora_linear_desc* desc, const void* X, const void* W, const void* A,
                            const void* B, void* H, float* U_save, void* ws, size_t ws_bytes, void* stream) {
    lora_status st = check_desc(desc, false);
    if (st != LORA_OK) return st;
    st = check_ptrs({{X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {H, "H"}}, {{U_save, "U_save"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{H, "H"}, {U_save, "U_save"}},
                        {{X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {H, "H"}, {U_save, "U_save"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(*desc, ws, ws_bytes);
    if (st != LORA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (desc->dtype == LORA_DTYPE_F32) return fwd_f32(*desc, false, X, W, nullptr, nullptr, nullptr, A, B, H, U_save, ws, s);
    return fwd_bf16(shape_of(*desc), false, X, W, nullptr, nullptr, nullptr, A, B, H, U_save, ws, s,
                    tuned_for(*desc, false));
}

lora_status lora_linear_bwd(const lora_linear_desc* desc, const void* dY, const void* X, const void* W,
                            const void* A, const void* B, const float* U_saved, void* dX, void* dA, void* dB,
                            void* ws, size_t ws_bytes, void* stream) {
    lora_status st = check_desc(desc, false);
    if (st != LORA_OK) return st;
    st = check_ptrs({{dY, "dY"}, {X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {dA, "dA"}, {dB, "dB"}},
                    {{U_saved, "U_saved"}, {dX, "dX"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                        {{dY, "dY"}, {X, "X"}, {W, "W"}, {A, "A"}, {B, "B"}, {U_saved, "U_saved"},
                         {dX, "dX"}, {dA, "dA"}, {dB, "dB"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(*desc, ws, ws_bytes);
    if (st != LORA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (desc->dtype == LORA_DTYPE_F32)
        return bwd_f32(*desc, false, dY, X, W, nullptr, nullptr, nullptr, A, B, U_saved, dX, dA, dB, ws, s);
    return bwd_bf16(shape_of(*desc), false, dY, X, W, nullptr, nullptr, nullptr, A, B, U_saved, dX, dA, dB, ws, s,
                    tuned_for(*desc, false));
}

lora_status lora_qlinear_fwd(const lora_linear_desc* desc, const void* X, const uint8_t* Wq, const uint16_t* absmax,
                             const float* codebook, const void* A, const void* B, void* H, float* U_save, void* ws,
                             size_t ws_bytes, void* stream) {
    lora_status st = check_desc(desc, true);
    if (st != LORA_OK) return st;
    st = check_ptrs({{X, "X"}, {Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {A, "A"}, {B, "B"}, {H, "H"}},
                    {{U_save, "U_save"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{H, "H"}, {U_save, "U_save"}},
                        {{X, "X"}, {Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {A, "A"}, {B, "B"},
                         {H, "H"}, {U_save, "U_save"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(*desc, ws, ws_bytes);
    if (st != LORA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (desc->dtype == LORA_DTYPE_F32) return fwd_f32(*desc, true, X, nullptr, Wq, absmax, codebook, A, B, H, U_save, ws, s);
    return fwd_bf16(shape_of(*desc), true, X, nullptr, Wq, absmax, codebook, A, B, H, U_save, ws, s,
                    tuned_for(*desc, true));
}

lora_status lora_qlinear_bwd(const lora_linear_desc* desc, const void* dY, const void* X, const uint8_t* Wq,
                             const uint16_t* absmax, const float* codebook, const void* A, const void* B,
                             const float* U_saved, void* dX, void* dA, void* dB, void* ws, size_t ws_bytes,
                             void* stream) {
    lora_status st = check_desc(desc, true);
    if (st != LORA_OK) return st;
    st = check_ptrs({{dY, "dY"}, {X, "X"}, {Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {A, "A"},
                     {B, "B"}, {dA, "dA"}, {dB, "dB"}},
                    {{U_saved, "U_saved"}, {dX, "dX"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                        {{dY, "dY"}, {X, "X"}, {Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {A, "A"},
                         {B, "B"}, {U_saved, "U_saved"}, {dX, "dX"}, {dA, "dA"}, {dB, "dB"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(*desc, ws, ws_bytes);
    if (st != LORA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (desc->dtype == LORA_DTYPE_F32)
        return bwd_f32(*desc, true, dY, X, nullptr, Wq, absmax, codebook, A, B, U_saved, dX, dA, dB, ws, s);
    return bwd_bf16(shape_of(*desc), true, dY, X, nullptr, Wq, absmax, codebook, A, B, U_saved, dX, dA, dB, ws, s,
                    tuned_for(*desc, true));
}

// ---------------------------------------------------------------- RMSNorm in front
// One launch of norm_prep_kernel: 1/rms of the M rows of X (none when X is
// NULL), and out = bf16(in diag(g)) for R rows of K columns.
static void launch_norm_prep(const uint16_t* X, float* inv, int64_t M, int64_t K, float eps, const uint16_t* in,
                             const uint16_t* g, uint16_t* out, int64_t R, hipStream_t s) {
    NormPrepArgs a{};
    a.X = X;
    a.inv = inv;
    a.M = (int)M;
    a.K = (int)K;
    a.rms_blocks = X ? (int)cdiv(M, 4) : 0;
    a.eps = eps;
    a.in = in;
    a.g = g;
    a.out = out;
    a.R = R;
    const int64_t blocks = a.rms_blocks + cdiv(R * K / 8, 256);
    if (X) LAUNCH("norm_prep", norm_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else LAUNCH("norm_fold", norm_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
}

static void launch_norm_dx(uint16_t* dX, const uint16_t* X, const float* inv, int64_t M, int64_t K, hipStream_t s) {
    const dim3 grid((unsigned)cdiv(M, 4));
    if (K <= 8 * kRowChunk) LAUNCH("norm_dx", norm_dx_kernel<8>, grid, dim3(256), 0, s, dX, X, inv, (int)M, (int)K);
    else if (K <= 16 * kRowChunk)
        LAUNCH("norm_dx", norm_dx_kernel<16>, grid, dim3(256), 0, s, dX, X, inv, (int)M, (int)K);
    else LAUNCH("norm_dx", norm_dx_kernel<0>, grid, dim3(256), 0, s, dX, X, inv, (int)M, (int)K);
}

static lora_status check_eps(float eps);

static lora_status check_norm(const lora_linear_desc* desc, float eps) {
    lora_status st = check_desc(desc, false);
    if (st != LORA_OK) return st;
    if (desc->dtype != LORA_DTYPE_BF16) return fail(LORA_ERR_UNSUPPORTED, "the RMSNorm path is bf16 only");
    return check_eps(eps);
}

static Shape norm_shape(const lora_linear_desc& d) {
    Shape s = shape_of(d);
    s.norm = true;
    return s;
}

lora_status lora_norm_linear_workspace_size(const lora_linear_desc* desc, size_t* bytes) {
    if (!bytes) return fail(LORA_ERR_INVALID_ARG, "bytes is NULL");
    lora_status st = check_norm(desc, 0.f);
    if (st != LORA_OK) return st;
    *bytes = make_plan(norm_shape(*desc)).total;
    return ok();
}

lora_status lora_transpose_weight(const void* W, int64_t N, int64_t K, void* Wt, void* stream) {
    if (N <= 0 || K <= 0) return fail(LORA_ERR_INVALID_ARG, "N, K must be positive");
    if (N % 8 || K % 8) return fail(LORA_ERR_UNSUPPORTED, "N and K must be multiples of 8 (N=%lld, K=%lld)",
                                    (long long)N, (long long)K);
    if (N * K > kMaxElems) return fail(LORA_ERR_UNSUPPORTED, "W has 2^31 or more elements");
    lora_status st = check_ptrs({{W, "W"}, {Wt, "Wt"}}, {});
    if (st != LORA_OK) return st;
    if (W == Wt) return fail(LORA_ERR_INVALID_ARG, "output Wt aliases W");
    const dim3 grid((unsigned)cdiv(K, 64), (unsigned)cdiv(N, 64));
    LAUNCH("transpose_weight", transpose_weight_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
           static_cast<const uint16_t*>(W), static_cast<uint16_t*>(Wt), (int)N, (int)K);
    LAUNCH_CHECK("transpose_weight");
    return ok();
}

lora_status lora_fold_norm_weight(const void* W, const void* g, int64_t N, int64_t K, void* W_out, void* stream) {
    if (N <= 0 || K <= 0) return fail(LORA_ERR_INVALID_ARG, "N, K must be positive");
    if (K % 8) return fail(LORA_ERR_UNSUPPORTED, "K must be a multiple of 8 (K=%lld)", (long long)K);
    if (N * K > kMaxElems) return fail(LORA_ERR_UNSUPPORTED, "W has 2^31 or more elements");
    lora_status st = check_ptrs({{W, "W"}, {g, "g"}, {W_out, "W_out"}}, {});
    if (st != LORA_OK) return st;
    if (W_out == g) return fail(LORA_ERR_INVALID_ARG, "output W_out aliases g");
    hipStream_t s = static_cast<hipStream_t>(stream);
    launch_norm_prep(nullptr, nullptr, 0, K, 0.f, static_cast<const uint16_t*>(W), static_cast<const uint16_t*>(g),
                     static_cast<uint16_t*>(W_out), N, s);
    LAUNCH_CHECK("norm_prep");
    return ok();
}

// The RMSNorm path for one layer or a group sharing the input (d.norm set).
static lora_status norm_fwd(const Shape& d, const void* X, const void* g, const void* W_g, const void* A,
                            const void* B, void* H, float* U_save, float* inv_rms_save, void* ws, size_t ws_bytes,
                            float eps, void* stream) {
    lora_status st = check_ptrs({{X, "X"}, {g, "g"}, {W_g, "W_g"}, {A, "A"}, {B, "B"}, {H, "H"}},
                                {{U_save, "U_save"}, {inv_rms_save, "inv_rms_save"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{H, "H"}, {U_save, "U_save"}, {inv_rms_save, "inv_rms_save"}},
                        {{X, "X"}, {g, "g"}, {W_g, "W_g"}, {A, "A"}, {B, "B"}, {H, "H"}, {U_save, "U_save"},
                         {inv_rms_save, "inv_rms_save"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(d, ws, ws_bytes);
    if (st != LORA_OK) return st;
    const Plan plan = make_plan(d);
    char* const wsb = static_cast<char*>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* const inv = inv_rms_save ? inv_rms_save : reinterpret_cast<float*>(wsb + plan.off_inv);
    uint16_t* const Ag = reinterpret_cast<uint16_t*>(wsb + plan.off_ag);
    const uint16_t* const X16 = static_cast<const uint16_t*>(X);
    const int64_t rg = d.rg();
    launch_norm_prep(X16, inv, d.M, d.K, eps, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(g), Ag,
                     rg, s);
    LAUNCH_CHECK("norm_prep");
    return fwd_bf16(d, false, X, W_g, nullptr, nullptr, nullptr, Ag, B, H, U_save, ws, s, Tuning{}, inv);
}

static lora_status norm_bwd(const Shape& d, const void* dY, const void* X, const void* g, const void* W_g,
                            const void* A, const void* B, const float* U_saved, const float* inv_rms_saved, void* dX,
                            void* dA, void* dB, void* ws, size_t ws_bytes, float eps, void* stream) {
    lora_status st = check_ptrs({{dY, "dY"}, {X, "X"}, {g, "g"}, {W_g, "W_g"}, {A, "A"}, {B, "B"}, {dA, "dA"},
                                 {dB, "dB"}},
                                {{U_saved, "U_saved"}, {inv_rms_saved, "inv_rms_saved"}, {dX, "dX"}});
    if (st != LORA_OK) return st;
    st = check_no_alias({{dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                        {{dY, "dY"}, {X, "X"}, {g, "g"}, {W_g, "W_g"}, {A, "A"}, {B, "B"}, {U_saved, "U_saved"},
                         {inv_rms_saved, "inv_rms_saved"}, {dX, "dX"}, {dA, "dA"}, {dB, "dB"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(d, ws, ws_bytes);
    if (st != LORA_OK) return st;
    const Plan plan = make_plan(d);
    char* const wsb = static_cast<char*>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* const X16 = static_cast<const uint16_t*>(X);
    const uint16_t* const g16 = static_cast<const uint16_t*>(g);
    const int64_t rg = d.rg();
    // 1/rms (unless saved by the forward) and A diag(g) in one launch
    float* const inv_ws = reinterpret_cast<float*>(wsb + plan.off_inv);
    const float* const inv = inv_rms_saved ? inv_rms_saved : inv_ws;
    uint16_t* const Ag = reinterpret_cast<uint16_t*>(wsb + plan.off_ag);
    launch_norm_prep(inv_rms_saved ? nullptr : X16, inv_ws, d.M, d.K, eps, static_cast<const uint16_t*>(A), g16, Ag,
                     rg, s);
    LAUNCH_CHECK("norm_prep");
    // dY W_g + s V A_g into dX, dA = s g (inv V)^T X, dB = s dY^T U
    st = bwd_bf16(d, false, dY, X, W_g, nullptr, nullptr, nullptr, Ag, B, U_saved, dX, dA, dB, ws, s, Tuning{}, inv,
                  g16);
    if (st != LORA_OK) return st;
    if (dX) {
        // through the norm: dX = inv D - X (inv^3 / K) <D, X>, D = dY W_g + s V A_g
        launch_norm_dx(static_cast<uint16_t*>(dX), X16, inv, d.M, d.K, s);
        LAUNCH_CHECK("norm_dx");
    }
    return ok();
}

static lora_status check_eps(float eps) {
    if (!std::isfinite(eps) || eps < 0.f) return fail(LORA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    return LORA_OK;
}

lora_status lora_norm_linear_fwd(const lora_linear_desc* desc, float eps, const void* X, const void* g,
                                 const void* W_g, const void* A, const void* B, void* H, float* U_save,
                                 float* inv_rms_save, void* ws, size_t ws_bytes, void* stream) {
    lora_status st = check_norm(desc, eps);
    if (st != LORA_OK) return st;
    return norm_fwd(norm_shape(*desc), X, g, W_g, A, B, H, U_save, inv_rms_save, ws, ws_bytes, eps, stream);
}

lora_status lora_norm_linear_bwd(const lora_linear_desc* desc, float eps, const void* dY, const void* X,
                                 const void* g, const void* W_g, const void* A, const void* B, const float* U_saved,
                                 const float* inv_rms_saved, void* dX, void* dA, void* dB, void* ws, size_t ws_bytes,
                                 void* stream) {
    lora_status st = check_norm(desc, eps);
    if (st != LORA_OK) return st;
    return norm_bwd(norm_shape(*desc), dY, X, g, W_g, A, B, U_saved, inv_rms_saved, dX, dA, dB, ws, ws_bytes, eps,
                    stream);
}

static Shape norm_group_shape(const lora_group_desc& gd) {
    Shape s = shape_of(gd);
    s.norm = true;
    return s;
}

lora_status lora_norm_group_workspace_size(const lora_group_desc* desc, size_t* bytes) {
    if (!bytes) return fail(LORA_ERR_INVALID_ARG, "bytes is NULL");
    lora_status st = check_group(desc);
    if (st != LORA_OK) return st;
    *bytes = make_plan(norm_group_shape(*desc)).total;
    return ok();
}

lora_status lora_norm_group_fwd(const lora_group_desc* desc, float eps, const void* X, const void* g,
                                const void* W_g, const void* A, const void* B, void* H, float* U_save,
                                float* inv_rms_save, void* ws, size_t ws_bytes, void* stream) {
    lora_status st = check_group(desc);
    if (st == LORA_OK) st = check_eps(eps);
    if (st != LORA_OK) return st;
    return norm_fwd(norm_group_shape(*desc), X, g, W_g, A, B, H, U_save, inv_rms_save, ws, ws_bytes, eps, stream);
}

lora_status lora_norm_group_bwd(const lora_group_desc* desc, float eps, const void* dY, const void* X,
                                const void* g, const void* W_g, const void* A, const void* B, const float* U_saved,
                                const float* inv_rms_saved, void* dX, void* dA, void* dB, void* ws, size_t ws_bytes,
                                void* stream) {
    lora_status st = check_group(desc);
    if (st == LORA_OK) st = check_eps(eps);
    if (st != LORA_OK) return st;
    return norm_bwd(norm_group_shape(*desc), dY, X, g, W_g, A, B, U_saved, inv_rms_saved, dX, dA, dB, ws, ws_bytes,
                    eps, stream);
}

lora_status lora_tune_linear(const lora_linear_desc* desc, int32_t quant, const void* X, const void* W,
                             const uint8_t* Wq, const uint16_t* absmax, const float* codebook, const void* A,
                             const void* B, void* H, float* U, const void* dY, void* dX, void* dA, void* dB, void* ws,
                             size_t ws_bytes, void* stream, int32_t reps, lora_tuned_config* chosen) {
    const bool q = quant != 0;
    lora_status st = check_desc(desc, q);
    if (st != LORA_OK) return st;
    if (desc->dtype != LORA_DTYPE_BF16) return fail(LORA_ERR_UNSUPPORTED, "only the bf16 path has launch parameters");
    if (desc->flags & LORA_FLAG_W_TRANSPOSED)
        return fail(LORA_ERR_UNSUPPORTED, "the tuner runs forward and backward with one W: no LORA_FLAG_W_TRANSPOSED");
    if (reps < 1 || reps > 100) return fail(LORA_ERR_INVALID_ARG, "reps = %d (1 .. 100)", (int)reps);
    st = check_ptrs({{X, "X"}, {A, "A"}, {B, "B"}, {H, "H"}, {U, "U"}, {dY, "dY"}, {dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                    {{W, "W"}, {Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}});
    if (st != LORA_OK) return st;
    if (q ? (!Wq || !absmax || !codebook) : !W)
        return fail(LORA_ERR_INVALID_ARG, q ? "Wq, absmax and codebook are needed" : "W is NULL");
    st = check_no_alias({{H, "H"}, {U, "U"}, {dX, "dX"}, {dA, "dA"}, {dB, "dB"}},
                        {{X, "X"}, {W, "W"}, {Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {A, "A"},
                         {B, "B"}, {H, "H"}, {U, "U"}, {dY, "dY"}, {dX, "dX"}, {dA, "dA"}, {dB, "dB"}, {ws, "ws"}});
    if (st != LORA_OK) return st;
    st = check_ws(*desc, ws, ws_bytes);
    if (st != LORA_OK) return st;
    std::string arch;
    int cus = 0;
    if (!current_device_info(arch, cus)) return fail(LORA_ERR_HIP, "no current HIP device");
    Shape d = shape_of(*desc);
    d.flags &= ~LORA_FLAG_ACCUM_GRADS;          // repeated runs must not accumulate
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return fail(LORA_ERR_HIP, "hipEventCreate failed");
    }
    lora_status err = LORA_OK;
    auto fwd = [&](const Tuning& tn) {
        return fwd_bf16(d, q, X, W, Wq, absmax, codebook, A, B, H, U, ws, s, tn);
    };
    auto bwd = [&](const Tuning& tn) {
        return bwd_bf16(d, q, dY, X, W, Wq, absmax, codebook, A, B, U, dX, dA, dB, ws, s, tn);
    };
    // Median times (us) of the candidates, measured round-robin (one run of each
    // per round, after a warm-up round) so that the clock's drift under load
    // affects all of them alike; candidate 0 is the built-in rules.
    auto medians = [&](const std::vector<Tuning>& cand, auto&& run) {
        std::vector<std::vector<float>> t(cand.size());
        for (int round = 0; round <= reps && err == LORA_OK; ++round) {
            for (size_t i = 0; i < cand.size() && err == LORA_OK; ++i) {
                if (hipEventRecord(e0, s) != hipSuccess) {
                    err = fail(LORA_ERR_HIP, "hipEventRecord failed");
                    break;
                }
                err = run(cand[i]);
                if (err != LORA_OK) break;
                float ms = 0.f;
                if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                    hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
                    err = fail(LORA_ERR_HIP, "timing a candidate failed");
                    break;
                }
                if (round > 0) t[i].push_back(ms * 1e3f);
            }
        }
        std::vector<float> med(cand.size(), 0.f);
        for (size_t i = 0; i < cand.size(); ++i) {
            if (t[i].empty()) continue;
            std::sort(t[i].begin(), t[i].end());
            med[i] = t[i][t[i].size() / 2];
        }
        return med;
    };
    // the candidate with the least median, unless it beats the built-in rules by less than 2 %
    auto pick = [](const std::vector<float>& med) {
        size_t b = 0;
        for (size_t i = 1; i < med.size(); ++i)
            if (med[i] < med[b]) b = i;
        return med[b] < 0.98f * med[0] ? b : 0;
    };
    auto same_split = [](const SplitPlan& a, const SplitPlan& b) {
        return a.first == b.first && a.split == b.split && a.kc == b.kc;
    };
    // distinct split modes of a GEMM (modes giving the same plan are one candidate)
    auto split_modes = [&](int64_t P, int64_t Qd, int64_t C) {
        std::vector<int> modes{0};
        std::vector<SplitPlan> seen{split_for(0, P, Qd, C)};
        for (int mode = 1; mode <= 3; ++mode) {
            const SplitPlan sp = split_for(mode, P, Qd, C);
            if (std::none_of(seen.begin(), seen.end(), [&](const SplitPlan& o) { return same_split(o, sp); })) {
                seen.push_back(sp);
                modes.push_back(mode);
            }
        }
        return modes;
    };
    // distinct divisors of a chunk count (1 first)
    auto divisors = [](int n) {
        std::vector<int> out{1};
        for (int div = 2; div <= 4; div *= 2)
            if (n / div >= 1 && n / div != n / (div / 2)) out.push_back(div);
        return out;
    };
    // forward: contraction split x the U pass's chunks (when U is streamed)
    std::vector<Tuning> fc;
    for (int mode : split_modes(d.M, d.N, d.K)) {
        const bool u_streamed = !gemm_in_tile(q, (int)d.r, split_for(mode, d.M, d.N, d.K));
        for (int zd : u_streamed ? divisors(z_chunks(d.M, d.K)) : std::vector<int>{1}) {
            Tuning c;
            c.fwd_split = mode;
            c.z_div_f = zd;
            fc.push_back(c);
        }
    }
    const std::vector<float> mf = medians(fc, fwd);
    const size_t bf = err == LORA_OK ? pick(mf) : 0;
    Tuning best = fc[bf];
    // backward: contraction split x adapter-gradient chunks x the V pass's chunks (when V is streamed)
    std::vector<Tuning> bc;
    for (int mode : split_modes(d.M, d.K, d.N)) {
        const bool v_streamed = !dx_in_tile(q, (int)d.r, split_for(mode, d.M, d.K, d.N));
        for (int rd : divisors(split_g(d).n_chunk))
            for (int zd : v_streamed ? divisors(z_chunks(d.M, d.N)) : std::vector<int>{1}) {
                Tuning c = best;
                c.bwd_split = mode;
                c.rank_div = rd;
                c.z_div_b = zd;
                bc.push_back(c);
            }
    }
    const std::vector<float> mb = err == LORA_OK ? medians(bc, bwd) : std::vector<float>(bc.size(), 0.f);
    const size_t bb = err == LORA_OK ? pick(mb) : 0;
    best = bc[bb];
    const float t_fwd = mf[bf], t_fwd_default = mf[0], t_bwd = mb[bb], t_bwd_default = mb[0];
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (err != LORA_OK) return err;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        g_tuned[tune_key(arch, cus, *desc, q)] = best;
        g_tune_any.store(true, std::memory_order_release);
    }
    if (chosen) {
        *chosen = lora_tuned_config{best.fwd_split, best.bwd_split, best.rank_div, best.z_div_f, best.z_div_b,
                                    t_fwd, t_bwd, t_fwd_default, t_bwd_default};
    }
    return ok();
}

lora_status lora_tuner_lookup(const char* arch, int32_t cus, const lora_linear_desc* desc, int32_t quant,
                              lora_tuned_config* out, int32_t* found) {
    if (!desc || !out || !found) return fail(LORA_ERR_INVALID_ARG, "desc, out and found must not be NULL");
    std::string a;
    int c = cus;
    if (arch) {
        a = arch;
    } else if (!current_device_info(a, c)) {
        return fail(LORA_ERR_HIP, "no current HIP device");
    }
    std::lock_guard<std::mutex> lock(g_tune_mu);
    const auto it = g_tuned.find(tune_key(a, c, *desc, quant != 0));
    *found = it != g_tuned.end();
    const Tuning t = *found ? it->second : Tuning{};
    *out = lora_tuned_config{t.fwd_split, t.bwd_split, t.rank_div, t.z_div_f, t.z_div_b, 0.f, 0.f, 0.f, 0.f};
    return ok();
}

lora_status lora_tuner_save(const char* path) {
    if (!path) return fail(LORA_ERR_INVALID_ARG, "path is NULL");
    FILE* f = std::fopen(path, "w");
    if (!f) return fail(LORA_ERR_INVALID_ARG, "cannot write %s", path);
    std::fprintf(f, "# lora tuning cache v1: arch cus M K N r quant fwd_split bwd_split rank_div z_div_fwd z_div_bwd\n");
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        for (const auto& kv : g_tuned) {
            const TuneKey& k = kv.first;
            const Tuning& t = kv.second;
            std::fprintf(f, "%s %d %lld %lld %lld %lld %d %d %d %d %d %d\n", k.arch.c_str(), k.cus, (long long)k.M,
                         (long long)k.K, (long long)k.N, (long long)k.r, k.quant, t.fwd_split, t.bwd_split, t.rank_div,
                         t.z_div_f, t.z_div_b);
        }
    }
    const bool bad = std::ferror(f) != 0;
    std::fclose(f);
    return bad ? fail(LORA_ERR_INVALID_ARG, "write error on %s", path) : ok();
}

lora_status lora_tuner_load(const char* path) {
    if (!path) return fail(LORA_ERR_INVALID_ARG, "path is NULL");
    FILE* f = std::fopen(path, "r");
    if (!f) return fail(LORA_ERR_INVALID_ARG, "cannot read %s", path);
    std::map<TuneKey, Tuning> read;
    char line[512];
    int lineno = 0;
    while (std::fgets(line, sizeof line, f)) {
        ++lineno;
        const char* p = line;
        while (*p == ' ' || *p == '\t') ++p;
        if (*p == '#' || *p == '\n' || *p == '\0') continue;
        char arch[64];
        int cus = 0, quant = 0;
        long long M = 0, K = 0, N = 0, r = 0;
        Tuning t;
        const int n = std::sscanf(p, "%63s %d %lld %lld %lld %lld %d %d %d %d %d %d", arch, &cus, &M, &K, &N, &r, &quant,
                                  &t.fwd_split, &t.bwd_split, &t.rank_div, &t.z_div_f, &t.z_div_b);
        if (n != 12 || cus <= 0 || M <= 0 || K <= 0 || N <= 0 || r <= 0 || (quant != 0 && quant != 1) ||
            !valid_tuning(t)) {
            std::fclose(f);
            return fail(LORA_ERR_INVALID_ARG, "%s:%d: not a tuning entry", path, lineno);
        }
        read[TuneKey{arch, cus, M, K, N, r, quant}] = t;
    }
    std::fclose(f);
    std::lock_guard<std::mutex> lock(g_tune_mu);
    for (const auto& kv : read) g_tuned[kv.first] = kv.second;
    g_tune_any.store(!g_tuned.empty(), std::memory_order_release);
    return ok();
}

void lora_tuner_clear(void) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned.clear();
    g_tune_any.store(false, std::memory_order_release);
}

lora_status lora_merge(const lora_linear_desc* desc, const void* W, const void* A, const void* B, void* W_out,
                       int32_t sign, void* stream) {
    if (!desc) return fail(LORA_ERR_INVALID_ARG, "desc is NULL");
    const lora_linear_desc& d = *desc;
    if (d.K <= 0 || d.N <= 0 || d.r <= 0)
        return fail(LORA_ERR_INVALID_ARG, "K, N, r must be positive (got %lld, %lld, %lld)", (long long)d.K,
                    (long long)d.N, (long long)d.r);
    if (d.dtype != LORA_DTYPE_BF16 && d.dtype != LORA_DTYPE_F32)
        return fail(LORA_ERR_INVALID_ARG, "unknown dtype %d", (int)d.dtype);
    if (!std::isfinite(d.alpha)) return fail(LORA_ERR_INVALID_ARG, "alpha is not finite");
    if (sign != 1 && sign != -1) return fail(LORA_ERR_INVALID_ARG, "sign must be +1 (merge) or -1 (unmerge), got %d", (int)sign);
    if (d.r > kMergeMaxR) return fail(LORA_ERR_UNSUPPORTED, "r = %lld exceeds %d", (long long)d.r, kMergeMaxR);
    if (d.K % 8) return fail(LORA_ERR_UNSUPPORTED, "K must be a multiple of 8 (K=%lld)", (long long)d.K);
    if (d.N * d.K > kMaxElems || d.r * d.K > kMaxElems || d.N * d.r > kMaxElems)
        return fail(LORA_ERR_UNSUPPORTED, "a matrix has 2^31 or more elements");
    if (cdiv(d.N, kMergeRows) > 65535) return fail(LORA_ERR_UNSUPPORTED, "N = %lld is too large", (long long)d.N);
    lora_status st = check_ptrs({{W, "W"}, {A, "A"}, {B, "B"}, {W_out, "W_out"}}, {});
    if (st != LORA_OK) return st;
    // in place (W_out == W) is allowed; otherwise W_out's bytes must not overlap W, A or B
    const size_t es = d.dtype == LORA_DTYPE_F32 ? 4 : 2;
    auto overlaps = [](const void* p, size_t pn, const void* q, size_t qn) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
        return a < b + qn && b < a + pn;
    };
    const size_t wn = (size_t)d.N * d.K * es;
    if (W_out != W && overlaps(W_out, wn, W, wn)) return fail(LORA_ERR_INVALID_ARG, "W_out overlaps W (not in place)");
    if (overlaps(W_out, wn, A, (size_t)d.r * d.K * es)) return fail(LORA_ERR_INVALID_ARG, "W_out overlaps A");
    if (overlaps(W_out, wn, B, (size_t)d.N * d.r * es)) return fail(LORA_ERR_INVALID_ARG, "W_out overlaps B");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)cdiv(d.K, kMergeCols), (unsigned)cdiv(d.N, kMergeRows));
    const float scale = (float)sign * (d.alpha / (float)d.r);
    if (d.dtype == LORA_DTYPE_BF16 && d.r >= 16) {
        // MFMA form: from r ~ 16 the rank-r sum costs the VALU form more than its 4 bytes per weight
        const uint16_t *W16 = static_cast<const uint16_t*>(W), *A16 = static_cast<const uint16_t*>(A),
                       *B16 = static_cast<const uint16_t*>(B);
        uint16_t* const O16 = static_cast<uint16_t*>(W_out);
#define MERGE_MFMA(RP) LAUNCH("lora_merge", (lora_merge_mfma<RP>), grid, dim3(256), 0, s, W16, A16, B16, O16, \
                             (int)d.N, (int)d.K, (int)d.r, scale)
        switch ((d.r + 31) / 32) {
            case 1: MERGE_MFMA(32); break;
            case 2: MERGE_MFMA(64); break;
            case 3: MERGE_MFMA(96); break;
            default: MERGE_MFMA(128); break;
        }
#undef MERGE_MFMA
    } else if (d.dtype == LORA_DTYPE_F32)
        LAUNCH("lora_merge", (lora_merge_kernel<true>), grid, dim3(256), 0, s, W, A, B, W_out, (int)d.N, (int)d.K,
                           (int)d.r, scale);
    else
        LAUNCH("lora_merge", (lora_merge_kernel<false>), grid, dim3(256),
                           (size_t)d.r * (kMergeCols + kMergeRows) * sizeof(uint16_t), s, W, A, B, W_out, (int)d.N,
                           (int)d.K, (int)d.r, scale);
    LAUNCH_CHECK("lora_merge");
    return ok();
}

lora_status lora_dequant4(const uint8_t* Wq, const uint16_t* absmax, const float* codebook, int64_t N, int64_t K,
                          int32_t out_dtype, void* W_out, void* stream) {
    if (N <= 0 || K <= 0) return fail(LORA_ERR_INVALID_ARG, "N, K must be positive");
    if (K % 64) return fail(LORA_ERR_UNSUPPORTED, "K must be a multiple of 64");
    if (N * K > kMaxElems) return fail(LORA_ERR_UNSUPPORTED, "W has 2^31 or more elements");
    if (out_dtype != LORA_DTYPE_BF16 && out_dtype != LORA_DTYPE_F32)
        return fail(LORA_ERR_INVALID_ARG, "unknown out_dtype %d", (int)out_dtype);
    lora_status st = check_ptrs({{Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {W_out, "W_out"}}, {});
    if (st != LORA_OK) return st;
    st = check_no_alias({{W_out, "W_out"}}, {{Wq, "Wq"}, {absmax, "absmax"}, {codebook, "codebook"}, {W_out, "W_out"}});
    if (st != LORA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // groups of 8 weights; at most 16 workgroups per CU, grid-stride beyond that
    const int n_groups = (int)(N * K / 8);
    const dim3 grid((unsigned)std::min<int64_t>(cdiv(n_groups, 256), 256 * 16));
    if (out_dtype == LORA_DTYPE_F32)
        LAUNCH("dequant4", (dequant4_kernel<true>), grid, dim3(256), 0, s, Wq, absmax, codebook, W_out, n_groups);
    else
        LAUNCH("dequant4", (dequant4_kernel<false>), grid, dim3(256), 0, s, Wq, absmax, codebook, W_out, n_groups);
    LAUNCH_CHECK("dequant4");
    return ok();
}

}  // extern "C"
