// Byte ranges of the buffer resources the kernels build.
//
// A buffer resource describes [base, base + range) with a 32-bit range, and a
// load whose offset lands past it returns zeros.  Every kernel therefore
// builds its resources from a base near the data one workgroup (or one step)
// touches, so that the range stays below 2^31 bytes for every descriptor the
// C ABI accepts, and the out-of-range marker offset 2^31 can never be a valid
// offset.  The same functions are used by the kernels when they build the
// resources and by lora_linear_buffer_ranges, which lists the worst case of
// each one for a descriptor (host tests check them against 2^31 - 1).
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lora {

constexpr uint64_t kMaxRange = 0x7FFFFFFFu;          // largest range a resource can describe
constexpr int kSideBlock = 128;                      // token block of the rank planes (see zt_index)

__host__ __device__ inline int64_t rmin64(int64_t a, int64_t b) { return a < b ? a : b; }

// Rows [row0, row0 + rows) of a row-major bf16 matrix with C columns, clipped
// to its `total` rows: the GEMM's operand panels (rows = 256), rank_z_lds's Y
// block (128) and one rank_stream step (TM).
__host__ __device__ inline uint64_t panel_bytes(int64_t total, int64_t row0, int64_t rows, int64_t C) {
    return (uint64_t)rmin64(total - row0, rows) * (uint64_t)C * 2u;
}

// Rows [row0, row0 + rows) of a bf16 matrix with C used columns and row stride
// ld, clipped to its `total` rows (the last row only up to C).
__host__ __device__ inline uint64_t strided_panel_bytes(int64_t total, int64_t row0, int64_t rows, int64_t C,
                                                        int64_t ld) {
    return ((uint64_t)(rmin64(total - row0, rows) - 1) * (uint64_t)ld + (uint64_t)C) * 2u;
}

// Input-gradient GEMM, W tile of one stage: rows c0 .. c0 + 63 of W [C][Q]
// from column q0 on (the last row only up to Q).
__host__ __device__ inline uint64_t gemm_wt_stage_bytes(int64_t C, int64_t Q, int64_t c0, int64_t q0) {
    const int64_t rows_left = rmin64(C - c0, 64) < 1 ? 1 : rmin64(C - c0, 64);
    return (uint64_t)(rows_left - 1) * (uint64_t)Q * 2u + (uint64_t)(Q - q0) * 2u;
}

// rank_stream, Y tile of one step: rows m0 .. m0 + TM - 1 of Y [M][C] (row
// stride ld) from column c0 on (the last row only up to C).
__host__ __device__ inline uint64_t stream_y_bytes(int64_t M, int64_t C, int64_t m0, int64_t c0, int64_t TM,
                                                   int64_t ld) {
    return (uint64_t)(rmin64(M - m0, TM) - 1) * (uint64_t)ld * 2u + (uint64_t)(C - c0) * 2u;
}

// Rank planes (bf16 hi / lo of Z^T for the adapter gradients), token-block
// major: element (j, m) of an [r][Mp] plane sits at zt_index(j, m, r), i.e.
// blocks of 128 tokens, each holding its r rows of 128 consecutive tokens.
// One rank_stream step then reads one contiguous block, whatever M is.
__host__ __device__ inline size_t zt_index(int64_t j, int64_t m, int64_t r) {
    return ((size_t)(m / kSideBlock) * (size_t)r + (size_t)j) * kSideBlock + (size_t)(m % kSideBlock);
}

// rank_stream, side tile of one step: rank rows j0 .. j0 + rl - 1 of one token
// block, the first row from token offset `col` (0, or 64 for the second half
// of a block with 64-token steps), each row TM tokens.
__host__ __device__ inline uint64_t stream_side_bytes(int64_t rl, int64_t TM) {
    return ((uint64_t)(rl - 1) * kSideBlock + (uint64_t)TM) * 2u;
}

// 4-bit weights: codes [total][cols / 2] bytes (two per byte) and absmax
// [total][cols / 64] fp16.  One contraction stage of the 4-bit forward GEMM
// reads rows [row0, row0 + rows) from column col0 on, the last row only up to
// its end (256 weight rows at stage column c0).  The host lists them in
// int64_t; the kernel evaluates them in int (scalar instructions), exact
// because a weight matrix has fewer than 2^31 elements.
template <typename I>
__host__ __device__ inline I q4_rows(I total, I row0, I rows) {    // row0 < total
    return total - row0 < rows ? total - row0 : rows;
}
template <typename I>
__host__ __device__ inline I q4_code_bytes(I total, I row0, I rows, I cols, I col0) {
    return (q4_rows(total, row0, rows) - 1) * (cols / 2) + (cols - col0) / 2;
}
template <typename I>
__host__ __device__ inline I q4_absmax_bytes(I total, I row0, I rows, I cols, I col0) {
    return ((q4_rows(total, row0, rows) - 1) * (cols / 64) + (cols - col0) / 64) * 2;
}

// Small whole operands: A [r][K], B [N][r], B^T [r][N] (bf16).
__host__ __device__ inline uint64_t whole_bytes(int64_t rows, int64_t cols) {
    return (uint64_t)rows * (uint64_t)cols * 2u;
}

}  // namespace lora
