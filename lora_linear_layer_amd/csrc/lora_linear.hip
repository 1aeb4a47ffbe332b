// C ABI of the fused LoRA linear layer (declarations and contracts in
// include/lora_linear.h).  Host side: argument validation (before any HIP
// call), workspace planning, kernel selection and launches on the caller's
// stream.  No allocation, no state, no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "lora_linear.h"
#include "fused_gemm.hpp"
#include "lora_gemm.hpp"
#include "grad_splitm.hpp"
#include "f32_kernels.hpp"

using namespace lora;

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

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxDim = int64_t(1) << 21;   // K, N bound: one 256-row tile stays under 2 GB
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int rpad_of(int64_t r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

// Workspace layout for one descriptor (offsets in bytes from ws).
struct Plan {
    size_t off_v = 0, off_u = 0, off_pa = 0, off_pb = 0, off_zp = 0, total = 0;
    int n_mblk = 1, mblk_rows = 128;
    int max_zparts = 1;   // contraction chunks of the stand-alone rank-r products
};

// Chunks for a stand-alone rank-r product over C: enough workgroups (>= ~1024)
// to cover the HBM stream of Y, each chunk a multiple of 64.
int zparts_for(int64_t M, int64_t C) {
    const int64_t rows = cdiv(M, 64);
    int64_t n = cdiv(1024, rows);
    n = std::max<int64_t>(1, std::min<int64_t>(n, cdiv(C, 256)));
    return (int)n;
}

Plan make_plan(const lora_linear_desc& d) {
    Plan p;
    const size_t zbytes = align_up((size_t)d.M * d.r * sizeof(float));
    p.off_v = 0;
    p.off_u = zbytes;
    size_t cur = 2 * zbytes;
    if (d.dtype == LORA_DTYPE_BF16) {
        // enough m blocks that the two gradient problems give >= ~1024 workgroups
        const int64_t cblocks = cdiv(d.K, kGradCB) + cdiv(d.N, kGradCB);
        const int64_t max_mblk = cdiv(d.M, kGradMB);
        int64_t want = cdiv(1024, cblocks);
        if (want < 1) want = 1;
        if (want > max_mblk) want = max_mblk;
        const int64_t rows = cdiv(cdiv(d.M, want), kGradMB) * kGradMB;
        p.mblk_rows = (int)rows;
        p.n_mblk = (int)cdiv(d.M, rows);
        p.off_pa = cur;
        cur += align_up((size_t)p.n_mblk * d.K * d.r * sizeof(float));
        p.off_pb = cur;
        cur += align_up((size_t)p.n_mblk * d.N * d.r * sizeof(float));
        p.max_zparts = std::max(zparts_for(d.M, d.K), zparts_for(d.M, d.N));
        if (p.max_zparts > 1) {
            p.off_zp = cur;
            cur += align_up((size_t)p.max_zparts * d.M * d.r * sizeof(float));
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
    if ((d->flags & ~LORA_FLAG_ACCUM_GRADS) != 0)
        return fail(LORA_ERR_INVALID_ARG, "unknown flag bits 0x%x", (unsigned)d->flags);
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

lora_status check_ws(const lora_linear_desc& d, void* ws, size_t ws_bytes) {
    const size_t need = make_plan(d).total;
    if (ws_bytes < need)
        return fail(LORA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    if (need > 0 && !ws) return fail(LORA_ERR_INVALID_ARG, "ws is NULL but %zu bytes are needed", need);
    if (ws && !aligned16(ws)) return fail(LORA_ERR_MISALIGNED, "ws is not 16-byte aligned");
    return LORA_OK;
}

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
template <int MODE, int RPAD, bool ZIN>
void launch_fused_t(const FusedArgs& a, hipStream_t st) {
    const int tiles = (int)(cdiv(a.P, kBP) * cdiv(a.Q, kBQ));
    hipLaunchKernelGGL((fused_lora_gemm<MODE, RPAD, ZIN>), dim3(tiles), dim3(kThreads), 0, st, a);
}

template <int MODE>
void launch_fused(const FusedArgs& a, int rpad, bool zin, hipStream_t st) {
    if (zin) { launch_fused_t<MODE, 128, true>(a, st); return; }
    switch (rpad) {
        case 16: launch_fused_t<MODE, 16, false>(a, st); break;
        case 32: launch_fused_t<MODE, 32, false>(a, st); break;
        default: launch_fused_t<MODE, 64, false>(a, st); break;
    }
}

void launch_fused_mode(int mode, const FusedArgs& a, int rpad, bool zin, hipStream_t st) {
    switch (mode) {
        case kFwd: launch_fused<kFwd>(a, rpad, zin, st); break;
        case kDx: launch_fused<kDx>(a, rpad, zin, st); break;
        case kQFwd: launch_fused<kQFwd>(a, rpad, zin, st); break;
        default: launch_fused<kQDx>(a, rpad, zin, st); break;
    }
}

template <bool TRANS, int RPAD, bool ZIN>
void launch_gemm_t(const GemmArgs& a, hipStream_t st) {
    const int tiles = (int)(cdiv(a.P, g2::BP) * cdiv(a.Q, g2::BQ));
    hipLaunchKernelGGL((lora_gemm<TRANS, RPAD, ZIN>), dim3(tiles), dim3(g2::NT), 0, st, a);
}

// In-tile rank-r product for r <= 16 (the input gradient also needs r % 8 == 0,
// so that rows of B are whole 16-byte chunks); otherwise Z comes precomputed.
// In-tile rank-r product: the forward forms U = X A^T inside the GEMM for
// r <= 16.  The input gradient takes V = dY B from the stand-alone pass: its
// in-tile form needs the transposing reads of B next to those of W, which
// pushes the kernel past 256 VGPRs (measured: 197 us with V in-tile vs 174 us
// for pass + GEMM + adapter gradients on the 4096 x 4096 r=8 layer).
bool gemm_in_tile(bool trans, int r) { return r <= 16 && !trans; }

template <bool TRANS>
void launch_gemm(const GemmArgs& a, hipStream_t st) {
    if constexpr (!TRANS) {
        if (gemm_in_tile(TRANS, a.r)) { launch_gemm_t<TRANS, 16, false>(a, st); return; }
    }
    switch (rpad_of(a.r)) {
        case 16: launch_gemm_t<TRANS, 16, true>(a, st); break;
        case 32: launch_gemm_t<TRANS, 32, true>(a, st); break;
        case 64: launch_gemm_t<TRANS, 64, true>(a, st); break;
        default: launch_gemm_t<TRANS, 128, true>(a, st); break;
    }
}

void launch_skinny(const uint16_t* Y, const uint16_t* F, bool f_trans, float* Z, int P, int C, int r, hipStream_t st,
                   float* zpart) {
    const int parts = zpart ? zparts_for(P, C) : 1;
    const int chunk = (int)(cdiv(cdiv(C, parts), 64) * 64);
    const int n_parts = (int)cdiv(C, chunk);
    float* const out = n_parts > 1 ? zpart : Z;
    const dim3 grid((unsigned)cdiv(P, 64), (unsigned)n_parts);
    const int rp = rpad_of(r);
#define SK(RP)                                                                                            \
    if (f_trans) hipLaunchKernelGGL((skinny_rank<RP, true>), grid, dim3(256), 0, st, Y, F, out, P, C, r, chunk); \
    else hipLaunchKernelGGL((skinny_rank<RP, false>), grid, dim3(256), 0, st, Y, F, out, P, C, r, chunk);
    switch (rp) {
        case 16: SK(16) break;
        case 32: SK(32) break;
        case 64: SK(64) break;
        default: SK(128) break;
    }
#undef SK
    if (n_parts > 1) {
        const int64_t n = (int64_t)P * r;
        hipLaunchKernelGGL(skinny_sum, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, zpart, Z, n, n_parts);
    }
}

void launch_grad_partials(const GradArgs& g, int rpad, hipStream_t st) {
    const int cb = std::max(g.prob[0].n_cblk, g.n_prob > 1 ? g.prob[1].n_cblk : 0);
    const dim3 grid((unsigned)cb, (unsigned)g.n_mblk, (unsigned)g.n_prob);
    switch (rpad) {
        case 16: hipLaunchKernelGGL((grad_partials<16>), grid, dim3(256), 0, st, g); break;
        case 32: hipLaunchKernelGGL((grad_partials<32>), grid, dim3(256), 0, st, g); break;
        case 64: hipLaunchKernelGGL((grad_partials<64>), grid, dim3(256), 0, st, g); break;
        default: hipLaunchKernelGGL((grad_partials<128>), grid, dim3(256), 0, st, g); break;
    }
}

// ---------------------------------------------------------------- forward
lora_status fwd_bf16(const lora_linear_desc& d, int mode, const void* X, const void* W, const uint8_t* Wq,
                     const uint16_t* absmax, const float* codebook, const void* A, const void* B, void* H,
                     float* U_save, void* ws, hipStream_t st) {
    const Plan plan = make_plan(d);
    const int r = (int)d.r, rpad = rpad_of(r);
    float* const zpart = plan.max_zparts > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + plan.off_zp) : nullptr;
    if (mode == kFwd) {
        GemmArgs g{};
        g.L = static_cast<const uint16_t*>(X);
        g.R = static_cast<const uint16_t*>(W);
        g.F = static_cast<const uint16_t*>(A);
        g.E = static_cast<const uint16_t*>(B);
        g.Out = static_cast<uint16_t*>(H);
        g.Zsave = U_save;
        g.P = (int)d.M; g.Q = (int)d.N; g.C = (int)d.K; g.r = r;
        g.s = d.alpha / (float)d.r;
        if (!gemm_in_tile(false, r)) {
            float* U = U_save ? U_save : reinterpret_cast<float*>(static_cast<char*>(ws) + plan.off_u);
            launch_skinny(g.L, g.F, false, U, g.P, g.C, r, st, zpart);
            LAUNCH_CHECK("skinny_rank(U)");
            g.Zin = U;
            g.Zsave = nullptr;
        }
        launch_gemm<false>(g, st);
        LAUNCH_CHECK("lora_gemm(forward)");
        return ok();
    }
    const bool zin = rpad > 64;
    FusedArgs a{};
    a.L = static_cast<const uint16_t*>(X);
    a.R = static_cast<const uint16_t*>(W);
    a.Rq = Wq;
    a.Rabs = absmax;
    a.codebook = codebook;
    a.F = static_cast<const uint16_t*>(A);
    a.E = static_cast<const uint16_t*>(B);
    a.Out = static_cast<uint16_t*>(H);
    a.Zsave = U_save;
    a.P = (int)d.M; a.Q = (int)d.N; a.C = (int)d.K; a.r = r;
    a.s = d.alpha / (float)d.r;
    if (zin) {
        float* U = U_save ? U_save : reinterpret_cast<float*>(static_cast<char*>(ws) + plan.off_u);
        launch_skinny(a.L, a.F, false, U, a.P, a.C, r, st, zpart);
        LAUNCH_CHECK("skinny_rank(U)");
        a.Zin = U;
        a.Zsave = nullptr;
    }
    launch_fused_mode(mode, a, rpad, zin, st);
    LAUNCH_CHECK("fused_lora_gemm(forward)");
    return ok();
}

// ---------------------------------------------------------------- backward
lora_status bwd_bf16(const lora_linear_desc& d, bool quant, const void* dY, const void* X, const void* W,
                     const uint8_t* Wq, const uint16_t* absmax, const float* codebook, const void* A,
                     const void* B, const float* U_saved, void* dX, void* dA, void* dB, void* ws, hipStream_t st) {
    const Plan plan = make_plan(d);
    const int r = (int)d.r, rpad = rpad_of(r);
    const bool zin = rpad > 64;
    char* const wsb = static_cast<char*>(ws);
    float* const V = reinterpret_cast<float*>(wsb + plan.off_v);
    float* const zpart = plan.max_zparts > 1 ? reinterpret_cast<float*>(wsb + plan.off_zp) : nullptr;
    const uint16_t* const dY16 = static_cast<const uint16_t*>(dY);
    const uint16_t* const X16 = static_cast<const uint16_t*>(X);
    const uint16_t* const A16 = static_cast<const uint16_t*>(A);
    const uint16_t* const B16 = static_cast<const uint16_t*>(B);

    // 1. dX = dY W + s V A with V = dY B formed on chip (and saved for dA)
    if (dX && !quant) {
        GemmArgs g{};
        g.L = dY16;
        g.R = static_cast<const uint16_t*>(W);
        g.F = B16;
        g.E = A16;
        g.Out = static_cast<uint16_t*>(dX);
        g.Zsave = V;
        g.P = (int)d.M; g.Q = (int)d.K; g.C = (int)d.N; g.r = r;
        g.s = d.alpha / (float)d.r;
        if (!gemm_in_tile(true, r)) {
            launch_skinny(dY16, B16, true, V, g.P, g.C, r, st, zpart);
            LAUNCH_CHECK("skinny_rank(V)");
            g.Zin = V;
            g.Zsave = nullptr;
        }
        launch_gemm<true>(g, st);
        LAUNCH_CHECK("lora_gemm(dX)");
    } else if (dX) {
        FusedArgs a{};
        a.L = dY16;
        a.R = static_cast<const uint16_t*>(W);
        a.Rq = Wq; a.Rabs = absmax; a.codebook = codebook;
        a.F = B16;
        a.E = A16;
        a.Out = static_cast<uint16_t*>(dX);
        a.Zsave = V;
        a.P = (int)d.M; a.Q = (int)d.K; a.C = (int)d.N; a.r = r;
        a.s = d.alpha / (float)d.r;
        if (zin) {
            launch_skinny(dY16, B16, true, V, a.P, a.C, r, st, zpart);
            LAUNCH_CHECK("skinny_rank(V)");
            a.Zin = V;
            a.Zsave = nullptr;
        }
        launch_fused_mode(quant ? kQDx : kDx, a, rpad, zin, st);
        LAUNCH_CHECK("fused_lora_gemm(dX)");
    } else {
        launch_skinny(dY16, B16, true, V, (int)d.M, (int)d.N, r, st, zpart);
        LAUNCH_CHECK("skinny_rank(V)");
    }
    // 2. U (saved by the forward, or rebuilt from X)
    const float* U = U_saved;
    if (!U) {
        float* Uw = reinterpret_cast<float*>(wsb + plan.off_u);
        launch_skinny(X16, A16, false, Uw, (int)d.M, (int)d.K, r, st, zpart);
        LAUNCH_CHECK("skinny_rank(U)");
        U = Uw;
    }
    // 3. split-M partials of dA (Y = X, Z = V) and dB (Y = dY, Z = U) in one launch
    GradArgs g{};
    g.prob[0] = GradProblem{X16, V, reinterpret_cast<float*>(wsb + plan.off_pa), (int)d.K, (int)cdiv(d.K, kGradCB)};
    g.prob[1] = GradProblem{dY16, U, reinterpret_cast<float*>(wsb + plan.off_pb), (int)d.N, (int)cdiv(d.N, kGradCB)};
    g.n_prob = 2;
    g.M = (int)d.M; g.r = r;
    g.mblk_rows = plan.mblk_rows; g.n_mblk = plan.n_mblk;
    launch_grad_partials(g, rpad, st);
    LAUNCH_CHECK("grad_partials");
    // 4. fixed-order reduction, scale, dtype, layout
    ReduceArgs ra{};
    ra.prob[0] = ReduceProblem{g.prob[0].part, dA, (int)d.K, 1};
    ra.prob[1] = ReduceProblem{g.prob[1].part, dB, (int)d.N, 0};
    ra.n_prob = 2;
    ra.r = r; ra.n_mblk = plan.n_mblk;
    ra.s = d.alpha / (float)d.r;
    ra.f32_out = 0;
    ra.accumulate = (d.flags & LORA_FLAG_ACCUM_GRADS) ? 1 : 0;
    const int64_t most = std::max(d.K, d.N) * d.r;
    hipLaunchKernelGGL(grad_reduce, dim3((unsigned)cdiv(most, 256), 2), dim3(256), 0, st, ra);
    LAUNCH_CHECK("grad_reduce");
    return ok();
}

// ---------------------------------------------------------------- float32 mode
template <int RMODE>
void launch_f32_fused(const F32FusedArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)cdiv(a.Q, 64), (unsigned)cdiv(a.P, 64));
    hipLaunchKernelGGL((f32_fused<RMODE>), grid, dim3(256), 0, st, a);
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
    const Plan plan = make_plan(d);
    float* U = U_save ? U_save : reinterpret_cast<float*>(static_cast<char*>(ws) + plan.off_u);
    const int M = (int)d.M, K = (int)d.K, N = (int)d.N, r = (int)d.r;
    hipLaunchKernelGGL(f32_skinny, dim3((unsigned)cdiv((int64_t)M * r, 256)), dim3(256), 0, st,
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
    const Plan plan = make_plan(d);
    char* const wsb = static_cast<char*>(ws);
    float* const V = reinterpret_cast<float*>(wsb + plan.off_v);
    const int M = (int)d.M, K = (int)d.K, N = (int)d.N, r = (int)d.r;
    const float s = d.alpha / (float)d.r;
    const float* dYf = static_cast<const float*>(dY);
    const float* Xf = static_cast<const float*>(X);
    hipLaunchKernelGGL(f32_skinny, dim3((unsigned)cdiv((int64_t)M * r, 256)), dim3(256), 0, st,
                       dYf, static_cast<const float*>(B), V, M, N, r, 1);
    LAUNCH_CHECK("f32_skinny(V)");
    const float* U = U_saved;
    if (!U) {
        float* Uw = reinterpret_cast<float*>(wsb + plan.off_u);
        hipLaunchKernelGGL(f32_skinny, dim3((unsigned)cdiv((int64_t)M * r, 256)), dim3(256), 0, st,
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
    hipLaunchKernelGGL(f32_grad, dim3((unsigned)cdiv((int64_t)K * r, 256)), dim3(256), 0, st,
                       Xf, (const float*)V, static_cast<float*>(dA), M, K, r, s, 1, acc);
    LAUNCH_CHECK("f32_grad(dA)");
    hipLaunchKernelGGL(f32_grad, dim3((unsigned)cdiv((int64_t)N * r, 256)), dim3(256), 0, st,
                       dYf, U, static_cast<float*>(dB), M, N, r, s, 0, acc);
    LAUNCH_CHECK("f32_grad(dB)");
    return ok();
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

lora_status lora_linear_workspace_size(const lora_linear_desc* desc, size_t* bytes) {
    if (!bytes) return fail(LORA_ERR_INVALID_ARG, "bytes is NULL");
    lora_status st = check_desc(desc, false);
    if (st != LORA_OK) return st;
    *bytes = make_plan(*desc).total;
    return ok();
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
    return fwd_bf16(*desc, kFwd, X, W, nullptr, nullptr, nullptr, A, B, H, U_save, ws, s);
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
    return bwd_bf16(*desc, false, dY, X, W, nullptr, nullptr, nullptr, A, B, U_saved, dX, dA, dB, ws, s);
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
    return fwd_bf16(*desc, kQFwd, X, nullptr, Wq, absmax, codebook, A, B, H, U_save, ws, s);
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
    return bwd_bf16(*desc, true, dY, X, nullptr, Wq, absmax, codebook, A, B, U_saved, dX, dA, dB, ws, s);
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
    const dim3 grid((unsigned)cdiv(N * (K / 16), 256));
    if (out_dtype == LORA_DTYPE_F32)
        hipLaunchKernelGGL((dequant4_kernel<true>), grid, dim3(256), 0, s, Wq, absmax, codebook, W_out, N, K);
    else
        hipLaunchKernelGGL((dequant4_kernel<false>), grid, dim3(256), 0, s, Wq, absmax, codebook, W_out, N, K);
    LAUNCH_CHECK("dequant4");
    return ok();
}

}  // extern "C"
