/*
 * lora_linear.h -- C ABI of the fused LoRA linear layer for AMD MI355X (gfx950).
 *
 * The layer (page "UnSloth加速库集成：编译级优化带来的性能飞跃", section
 * "为什么标准LoRA会慢？"): h = W x + B (A x), with A in R^{r x d_in},
 * B in R^{d_out x r} and r << d.  The adapter term is multiplied by the scale
 * s = alpha / r.  W is frozen: no gradient for W exists (page "ms-swift框架下
 * UnSloth与Liger-Kernel优化实战", section "UnSloth：让LoRA真正“低秩”起来").
 *
 * Row-major convention used by every entry point (one token per row):
 *   X  [M, K]  tokens x d_in          W  [N, K]  d_out x d_in (nn.Linear layout)
 *   A  [r, K]                         B  [N, r]
 *   H  [M, N] = X W^T + s (X A^T) B^T
 *   dY [M, N] upstream gradient       dX [M, K] = dY W + s (dY B) A
 *   dA [r, K] = s (dY B)^T X          dB [N, r] = s dY^T (X A^T)
 *   U  [M, r] = X A^T (float32; saved by the forward for the backward)
 * All matrices are dense with leading dimension equal to the row length.
 *
 * Memory: every pointer is caller-owned device memory (except `desc`, which is
 * host memory).  The library allocates nothing, keeps no state between calls
 * (apart from the optional kernel timer and the tuning cache below),
 * never modifies an input, and enqueues all work on `stream` (a hipStream_t
 * passed as void*; NULL means the null stream).  Calls return once the work is
 * enqueued; device faults surface at the caller's next synchronisation.
 * Outputs must not overlap inputs.  Device pointers must be 16-byte aligned.
 *
 * Errors: every function returns a lora_status.  Arguments are validated on
 * the host before any HIP call, so an error other than LORA_ERR_HIP means
 * nothing was enqueued.  lora_last_error() gives a text description of the
 * last failure on the calling thread.  Nothing aborts or throws across the ABI.
 */
#ifndef LORA_LINEAR_H
#define LORA_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
    LORA_OK = 0,
    LORA_ERR_INVALID_ARG = 1,        /* null pointer, non-positive size, bad dtype, aliasing, non-finite alpha */
    LORA_ERR_UNSUPPORTED = 2,        /* shape outside the supported range (see below) */
    LORA_ERR_MISALIGNED = 3,         /* a device pointer is not 16-byte aligned */
    LORA_ERR_WORKSPACE_TOO_SMALL = 4,/* ws_bytes < lora_linear_workspace_size() */
    LORA_ERR_HIP = 5                 /* a HIP launch failed; see lora_last_error() */
} lora_status;

typedef enum lora_dtype {
    LORA_DTYPE_BF16 = 0,  /* bf16 storage, float32 accumulation (the hot path) */
    LORA_DTYPE_F32 = 1    /* float32 storage and arithmetic (debug / checking mode) */
} lora_dtype;

/* flags */
#define LORA_FLAG_ACCUM_GRADS 0x1u   /* backward adds into dA, dB instead of overwriting */
/* The W argument of the backward entry points (lora_linear_bwd, _bwd_noalloc,
 * lora_group_bwd, lora_norm_linear_bwd, lora_norm_group_bwd) is W^T [K, N]
 * (stacked: [K, N_total]; behind a norm: W_g^T), made once from the frozen
 * weight with lora_transpose_weight; the forward entry points still take W
 * [N, K] and ignore the flag.  The input-gradient GEMM then reads its weight
 * operand like the forward reads W; results are bit-identical to the call
 * with W.  bf16 weights only (4-bit, float32 mode, the tuner:
 * LORA_ERR_UNSUPPORTED). */
#define LORA_FLAG_W_TRANSPOSED 0x2u

/*
 * Problem descriptor (host memory).
 *   M tokens, K = d_in, N = d_out, r = rank, alpha = lora_alpha (s = alpha/r).
 *   dtype applies to X, W, A, B, H, dY, dX, dA, dB.  U is always float32.
 * Supported range: 1 <= r <= 128; M, K, N >= 1; K % 8 == 0 and N % 8 == 0;
 * K, N <= 2^21; every matrix has fewer than 2^31 elements; the 4-bit entry
 * points also need K % 64 == 0.  Outside it: LORA_ERR_UNSUPPORTED.
 */
typedef struct lora_linear_desc {
    int64_t M, K, N, r;
    float alpha;
    int32_t dtype;    /* lora_dtype */
    uint32_t flags;   /* LORA_FLAG_* */
} lora_linear_desc;

/* Bytes of device workspace any fwd/bwd call with this descriptor needs
 * (the same figure for the plain and the 4-bit entry points).  May be 0.
 * The workspace holds the intermediates passed between the kernels of one
 * call (rank-r products, split partial sums); its contents on entry do not
 * matter, and calls that share one workspace must be ordered on one stream. */
lora_status lora_linear_workspace_size(const lora_linear_desc* desc, size_t* bytes);

/*
 * Forward, fused: H = X W^T + s (X A^T) B^T in one kernel (page "ms-swift高效
 * 微调组合：LoRA+UnSloth提速实践", section 1.2 "算子融合": Linear, LoRA_A,
 * LoRA_B and the add in a single launch).  For r <= 16 with 16-bit W the
 * rank-r product U = X A^T is formed on chip, inside the main product's K loop
 * (U_save is its only trip to HBM); for larger r and for 4-bit W a streamed
 * pass over X forms U first and the GEMM epilogue reads it.
 *   U_save: optional float32 [M, r]; when non-NULL receives U for the backward.
 *   ws:     device workspace of ws_bytes bytes (NULL allowed when 0 is needed).
 */
lora_status lora_linear_fwd(const lora_linear_desc* desc,
                            const void* X, const void* W, const void* A, const void* B,
                            void* H, float* U_save,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Backward (page "Unsloth — 微调 2-5x 加速", section "核心要点", item 2: the
 * product is re-associated as A(B dY) so that only [M, r] intermediates exist;
 * page "ms-swift高效微调组合：LoRA+UnSloth提速实践", section 1.2: adapter
 * gradients in closed form without autograd).
 *   dX = dY W + s (dY B) A        (NULL: skipped)
 *   dA = s (dY B)^T X,  dB = s dY^T U   (overwritten, or accumulated with
 *                                        LORA_FLAG_ACCUM_GRADS)
 *   U_saved: float32 [M, r] from lora_linear_fwd, or NULL to recompute it from X.
 * Reductions over tokens run in a fixed order: results are bitwise
 * reproducible from run to run.
 */
lora_status lora_linear_bwd(const lora_linear_desc* desc,
                            const void* dY, const void* X, const void* W,
                            const void* A, const void* B, const float* U_saved,
                            void* dX, void* dA, void* dB,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Backward without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving or training loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * lora_linear_bwd (bitwise the same outputs), except that the intermediates
 * live in a static device array of LORA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per device, held until the process ends.  Nothing is
 * allocated.  The array's contents on entry do not matter (nothing in it has
 * to start at zero); every call on a device shares that device's array, so
 * calls that overlap on one device race: order them on one stream.  The
 * stream must belong to the current device.  A descriptor whose backward
 * needs more than LORA_NOALLOC_SCRATCH_BYTES of intermediates (large M x r, or
 * many split-M partials) gets LORA_ERR_UNSUPPORTED before anything is enqueued.
 */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

lora_status lora_linear_bwd_noalloc(const lora_linear_desc* desc,
                                    const void* dY, const void* X, const void* W,
                                    const void* A, const void* B, const float* U_saved,
                                    void* dX, void* dA, void* dB, void* stream);

/*
 * Linears that share one input (page "ms-swift高效微调组合：LoRA+UnSloth提速实践",
 * section 1.2, the fused q_proj example, and section 2.3, LoRA on all linear
 * layers: the attention projections q, k, v read the same hidden states, and
 * so do the MLP's gate and up).  The members are stored stacked, in member
 * order: member m has N[m] output columns, and with n0 = N[0] + .. + N[m-1]
 *   X  [M, K]             the shared input
 *   W  [sum N, K]         rows n0 .. n0 + N[m] - 1: member m's frozen weight
 *   A  [n_members r, K]   rows m r .. m r + r - 1: member m's A
 *   B  [sum N, r]         rows n0 .. : member m's B
 *   H, dY [M, sum N]      columns n0 .. : member m's output / its gradient
 *   U  [M, n_members r]   columns m r .. : member m's U = X A_m^T (float32)
 *   dA, dB                as A, B
 * Forward: H_m = X W_m^T + s (X A_m^T) B_m^T for every member, in one GEMM over
 * the stacked W whose epilogue adds each member's own rank-r term, after one
 * streamed pass over X that forms all members' U.  Backward: the input
 * gradient of the shared X is the sum over the members,
 *   dX = sum_m (dY_m W_m + s (dY_m B_m) A_m)     (one GEMM contracting over all
 *                                                 sum N columns; NULL: skipped),
 * and dA_m = s (dY_m B_m)^T X, dB_m = s dY_m^T U_m per member (overwritten, or
 * accumulated with LORA_FLAG_ACCUM_GRADS).  s = alpha / r for every member.
 * Requirements: 1 <= n_members <= LORA_MAX_MEMBERS; every N[m] >= 8 and a
 * multiple of 8; 1 <= r <= 128 and n_members r <= LORA_MAX_GROUP_RANK; K % 8 == 0;
 * K, sum N <= 2^21; every matrix under 2^31 elements; dtype LORA_DTYPE_BF16
 * (LORA_ERR_UNSUPPORTED otherwise).  Memory, errors and the workspace as for
 * lora_linear_fwd / lora_linear_bwd (lora_group_workspace_size).
 */
#define LORA_MAX_MEMBERS 8
#define LORA_MAX_GROUP_RANK 192

typedef struct lora_group_desc {
    int64_t M, K, r;
    float alpha;
    int32_t dtype;                   /* lora_dtype: LORA_DTYPE_BF16 */
    uint32_t flags;                  /* LORA_FLAG_* */
    int32_t n_members;
    int64_t N[LORA_MAX_MEMBERS];     /* output columns of each member (the first n_members entries) */
} lora_group_desc;

lora_status lora_group_workspace_size(const lora_group_desc* desc, size_t* bytes);

lora_status lora_group_fwd(const lora_group_desc* desc,
                           const void* X, const void* W, const void* A, const void* B,
                           void* H, float* U_save,
                           void* ws, size_t ws_bytes, void* stream);

lora_status lora_group_bwd(const lora_group_desc* desc,
                           const void* dY, const void* X, const void* W,
                           const void* A, const void* B, const float* U_saved,
                           void* dX, void* dA, void* dB,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * RMSNorm in front of the layer (page "ms-swift框架下UnSloth与Liger-Kernel优化
 * 实战", section "关键融合策略解析", RMSNorm + Linear: the normalised input is
 * never written out and read back).  The layer is applied to
 *   Xn[m, k] = X[m, k] inv[m] g[k],   inv[m] = 1 / sqrt(mean_k X[m, k]^2 + eps),
 * with the norm weight g [K] (bf16) frozen like W.  g is folded into the frozen
 * weight once: lora_fold_norm_weight writes W_g = bf16(W diag(g)) ([N, K]; W_out
 * may be W itself).  The entry points then read the raw X:
 *   forward:  H = Xn W^T + s (Xn A^T) B^T, computed as inv (X W_g^T + s X (A diag g)^T B^T);
 *             U_save (optional) receives U = Xn A^T, inv_rms_save (optional,
 *             float32 [M]) receives inv for the backward;
 *   backward: dX = the gradient with respect to the raw X (through the norm),
 *             dA = s (dY B)^T Xn, dB = s dY^T U; U_saved / inv_rms_saved NULL:
 *             recomputed from X.  No gradient for g (frozen).
 * Shapes, flags, errors and ownership as for lora_linear_fwd / _bwd, with the
 * workspace of lora_norm_linear_workspace_size; eps >= 0; bf16 only
 * (LORA_ERR_UNSUPPORTED otherwise).
 */
/*
 * Wt = W^T: W [N, K] bf16 -> Wt [K, N] bf16, for LORA_FLAG_W_TRANSPOSED
 * (the frozen weight transposed once, kept beside W; the adapter's
 * re-associated backward of page "Unsloth — 微调 2-5x 加速", section "核心要点",
 * item 2, then reads it in the forward's layout).  N, K multiples of 8;
 * Wt must not alias W.  Enqueued on `stream`.
 */
lora_status lora_transpose_weight(const void* W, int64_t N, int64_t K, void* Wt, void* stream);

lora_status lora_fold_norm_weight(const void* W, const void* g, int64_t N, int64_t K, void* W_out, void* stream);

lora_status lora_norm_linear_workspace_size(const lora_linear_desc* desc, size_t* bytes);

lora_status lora_norm_linear_fwd(const lora_linear_desc* desc, float eps,
                                 const void* X, const void* g, const void* W_g, const void* A, const void* B,
                                 void* H, float* U_save, float* inv_rms_save,
                                 void* ws, size_t ws_bytes, void* stream);

lora_status lora_norm_linear_bwd(const lora_linear_desc* desc, float eps,
                                 const void* dY, const void* X, const void* g, const void* W_g,
                                 const void* A, const void* B, const float* U_saved, const float* inv_rms_saved,
                                 void* dX, void* dA, void* dB,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * RMSNorm in front of a group of linears that share the normalised input (the
 * q/k/v projections behind the attention norm, gate/up behind the MLP norm):
 * the same operation for every member of a lora_group_desc, with the stacked
 * layout of lora_group_fwd / _bwd; W_g is the stacked weight with g folded in
 * (lora_fold_norm_weight over all N_total rows) and dX is the gradient with
 * respect to the raw X of the summed members.  Workspace from
 * lora_norm_group_workspace_size; errors as for lora_group_fwd / _bwd plus
 * eps >= 0.
 */
lora_status lora_norm_group_workspace_size(const lora_group_desc* desc, size_t* bytes);

lora_status lora_norm_group_fwd(const lora_group_desc* desc, float eps,
                                const void* X, const void* g, const void* W_g, const void* A, const void* B,
                                void* H, float* U_save, float* inv_rms_save,
                                void* ws, size_t ws_bytes, void* stream);

lora_status lora_norm_group_bwd(const lora_group_desc* desc, float eps,
                                const void* dY, const void* X, const void* g, const void* W_g,
                                const void* A, const void* B, const float* U_saved, const float* inv_rms_saved,
                                void* dX, void* dA, void* dB,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * 4-bit frozen weight (page "Unsloth — 微调 2-5x 加速", section "核心要点",
 * item 3: 4-bit weights are dequantised inside the matmul, not copied out
 * first).  W is replaced by
 *   Wq       [N, K/2] uint8: element k in the low nibble of byte k/2 when k is
 *            even, in the high nibble when k is odd;
 *   absmax   [N, K/64] IEEE fp16 bit patterns, one per 64 consecutive k;
 *   codebook [16] float32 (device memory).
 * Weight value: bf16_rne(float32(codebook[code] * float32(absmax))) in bf16
 * mode; the float32 product itself in f32 mode.  Requires K % 64 == 0.
 */
lora_status lora_qlinear_fwd(const lora_linear_desc* desc,
                             const void* X, const uint8_t* Wq, const uint16_t* absmax,
                             const float* codebook, const void* A, const void* B,
                             void* H, float* U_save,
                             void* ws, size_t ws_bytes, void* stream);

lora_status lora_qlinear_bwd(const lora_linear_desc* desc,
                             const void* dY, const void* X, const uint8_t* Wq,
                             const uint16_t* absmax, const float* codebook,
                             const void* A, const void* B, const float* U_saved,
                             void* dX, void* dA, void* dB,
                             void* ws, size_t ws_bytes, void* stream);

/* Standalone dequantisation of the 4-bit format above into a dense W_out [N, K]
 * (out_dtype LORA_DTYPE_BF16 or LORA_DTYPE_F32).  Requires K % 64 == 0. */
lora_status lora_dequant4(const uint8_t* Wq, const uint16_t* absmax, const float* codebook,
                          int64_t N, int64_t K, int32_t out_dtype, void* W_out, void* stream);

/*
 * Merge / unmerge (page "ms-swift框架下UnSloth与Liger-Kernel优化实战", section
 * "设计权衡与最佳实践", item 4: before deployment the adapter is folded into
 * the base weight, so that inference engines see a plain linear layer):
 *   W_out = W + sign * s * B A        sign = +1 merge, -1 unmerge; s = alpha / r
 * from desc (K, N, r, alpha, dtype; M is not used).  W, W_out [N, K], A [r, K],
 * B [N, r] in desc->dtype; float32 arithmetic, one rounding to the dtype
 * (bf16 with r >= 16 forms the rank-r sum on the matrix cores, float32
 * accumulation; otherwise fused multiply-adds in increasing j).
 * W_out may be W itself (in place); otherwise its bytes must not overlap W, A
 * or B (LORA_ERR_INVALID_ARG).  Requires 1 <= r <= 128 and K % 8 == 0
 * (LORA_ERR_UNSUPPORTED); other invalid arguments as for the entry points above.
 */
lora_status lora_merge(const lora_linear_desc* desc, const void* W, const void* A, const void* B,
                       void* W_out, int32_t sign, void* stream);

/*
 * Buffer ranges (a check of the library's own addressing, host only; no HIP
 * call).  The bf16 kernels read their large operands through buffer resources,
 * whose range field holds at most 2^31 - 1 bytes; each resource is therefore
 * based near the rows one workgroup or one pipeline step reads.  This lists,
 * for the plain (quant = 0) or 4-bit (quant = 1) entry points and this
 * descriptor, every resource a forward or backward call may build: the kernel,
 * the operand and the largest range in bytes it asks for.  The range of every
 * entry stays at or below 2^31 - 1 for every descriptor the entry points
 * accept.  The float32 mode builds none (count 0).
 *   out:      caller-owned host array of `capacity` entries (may be NULL when
 *             capacity is 0); the strings are static.
 *   count:    receives the number of entries (also when it exceeds capacity;
 *             then only the first `capacity` are written).
 * Errors as for the descriptor checks of the entry points.
 */
typedef struct lora_buffer_range {
    const char* kernel;
    const char* operand;
    uint64_t bytes;
} lora_buffer_range;

lora_status lora_linear_buffer_ranges(const lora_linear_desc* desc, int32_t quant, lora_buffer_range* out,
                                      int32_t capacity, int32_t* count);

/*
 * Auto-tuning (page "UnSloth加速库集成：编译级优化带来的性能飞跃", section
 * "技术三：自动调优引擎（Auto-tuning）": the best launch configuration differs
 * with the GPU, the sequence length and the rank, so it is probed on the first
 * run and cached for reuse).  The tuned parameters of the bf16 path are
 *   fwd_split, bwd_split  contraction split of the forward / input-gradient
 *                         GEMM: 0 the built-in rule (the same as 3), 1 no
 *                         split, 2 split outputs of under 128 tiles only, 3 also
 *                         split the tiles of a last round at most half full;
 *   rank_div              the adapter-gradient pass's token chunks: the
 *                         built-in count divided by 1, 2 or 4;
 *   z_div_fwd, z_div_bwd  the streamed U (forward) / V and U (backward) passes'
 *                         contraction chunks, divided likewise.
 * Every choice fits the workspace lora_linear_workspace_size gives, and every
 * choice computes the same result up to the order of float32 additions.
 *
 * lora_tune_linear runs the forward and the backward of a plain layer (quant 0:
 * W; quant 1: Wq, absmax, codebook) with every candidate, round-robin, reps
 * rounds after one warm-up round (HIP events on `stream`; the call blocks until
 * they finish), keeps per direction the candidate with the least median time
 * if it beats the built-in rules by at least 2 % (else the built-in rules),
 * and stores the choice in the process-wide cache
 * under (device architecture, compute units, M, K, N, r, quant).  From then on
 * lora_linear_fwd / _bwd and lora_qlinear_fwd / _bwd on such a device with
 * such a descriptor use it (the grouped and allocation-free entry points keep
 * the built-in rules).  It overwrites H, U, dX, dA and dB (dA, dB are
 * overwritten even with LORA_FLAG_ACCUM_GRADS).  `chosen` (optional) receives
 * the choice and the median times in µs of it and of the built-in rules.
 * dtype must be LORA_DTYPE_BF16.
 *
 * lora_tuner_save writes the cache as text (one line per entry: arch cus M K N
 * r quant fwd_split bwd_split rank_div z_div_fwd z_div_bwd; '#' starts a
 * comment); lora_tuner_load merges such a file into it (LORA_ERR_INVALID_ARG
 * names the first malformed line; nothing is merged then); lora_tuner_clear
 * empties it; lora_tuner_lookup reports the entry for a descriptor on the
 * named architecture and compute-unit count (arch NULL: the current device).
 * The cache is shared by all threads; tuning and calls that use it may
 * overlap.
 */
typedef struct lora_tuned_config {
    int32_t fwd_split, bwd_split, rank_div, z_div_fwd, z_div_bwd;
    float fwd_us, bwd_us;                   /* chosen configuration, median */
    float default_fwd_us, default_bwd_us;   /* built-in rules, median */
} lora_tuned_config;

lora_status lora_tune_linear(const lora_linear_desc* desc, int32_t quant,
                             const void* X, const void* W, const uint8_t* Wq, const uint16_t* absmax,
                             const float* codebook, const void* A, const void* B,
                             void* H, float* U, const void* dY, void* dX, void* dA, void* dB,
                             void* ws, size_t ws_bytes, void* stream, int32_t reps,
                             lora_tuned_config* chosen);
lora_status lora_tuner_lookup(const char* arch, int32_t cus, const lora_linear_desc* desc, int32_t quant,
                              lora_tuned_config* out, int32_t* found);
lora_status lora_tuner_save(const char* path);
lora_status lora_tuner_load(const char* path);
void lora_tuner_clear(void);

/*
 * Kernel timer (a profiling aid for callers that time the kernels inside one
 * call).  When set, every entry point calls
 *   fn(user, kernel, stream, &start, &stop)
 * on the calling thread right before it enqueues each kernel, with a static
 * kernel label ("lora_gemm forward", "lora_gemm dX", "rank_stream",
 * "grad_final", ...) and the stream passed to the entry point.  fn may set
 * start and stop to events (hipEvent_t, created by the caller, as void*); the
 * library attaches them to that kernel's dispatch (hipExtLaunchKernel), so
 * they record the kernel's own start and end and add no commands between the
 * kernels.  Left NULL, the kernel launches untimed.  fn(NULL) removes the
 * timer.  It is the library's only process-wide setting: set or clear it
 * while no other thread is inside the library.
 */
typedef void (*lora_kernel_timer)(void* user, const char* kernel, void* stream, void** start_event,
                                  void** stop_event);

void lora_set_kernel_timer(lora_kernel_timer fn, void* user);

/* Static text for a status code. */
const char* lora_status_string(lora_status status);

/* Text of the last failure on the calling thread ("" if none). */
const char* lora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_LINEAR_H */
