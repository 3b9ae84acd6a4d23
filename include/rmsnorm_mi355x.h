/*
 * rmsnorm_mi355x — batch-invariant RMSNorm forward and backward for one
 * MI355X (gfx950), as a C ABI over plain device pointers.
 *
 * What is computed (pages by title; the section or equation named):
 *  - Megatron-LM PR "Fix the batch-invariant RMSNorm forward and its input
 *    gradient", "What does this PR do?": item 1 (the zero-centred offset,
 *    added after the cast to fp32, in the forward as in the backward) and
 *    item 2 (the input gradient dx_k = g_k w_k r - (r^3 x_k / D) sum_i g_i
 *    x_i w_i, with the weight entering once per term; the weight gradient).
 *  - RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel":
 *    the +1 is an fp32 operation; the SiLU-gated norm with the weight
 *    multiply in fp32; the backward takes the forward's saved rstd.
 *  - RL-Kernel PR "[DSv4][P1-5] rmsnorm_residual", "Summary" and
 *    "Implementation": output RMSNorm(x) plus a byte copy of x (not
 *    RMSNorm(x + residual)); bf16 activations, fp32 gamma, fp32 saved inverse
 *    RMS, bf16 dx and fp32 dgamma; r = rsqrt(mean(x^2) + eps),
 *    y = (x * r) * gamma; no atomics, split-K or stream-K; the residual
 *    branch's gradient is added to dx (review comment).
 *  - TransformerEngine issue "Expose Batch Invariant Kernels", sections 1-3
 *    and the checks table: a row's result must not depend on the batch it
 *    sits in; the reduction layout may depend on the row length only; an
 *    unsupported input is rejected, never sent silently down another path.
 *
 * Precision contract. x, y, dx, g, z, dz and residual tensors are bf16,
 * passed as raw uint16_t bits (bf16 or fp16 through the _dt entry points).
 * gamma, rstd and dgamma are fp32 (gamma also bf16 / fp16 through _dt). Per
 * row:
 *   ss   = sum_j x_j^2: fp32 squares added in fp64 along a fixed reduction
 *          tree chosen by D alone, rounded to fp32 once
 *   r    = 1/sqrt(ss / D + eps): fp32 division and addition, the reciprocal
 *          square root in fp64 and rounded to fp32 once; stored in rstd
 *   w_j  = gamma_j, or gamma_j + 1.0f when zero_centered_gamma != 0
 *   y_j  = bf16_rne((x_j * r) * w_j)                (two fp32 products)
 *   gated: out_j = bf16_rne(((x_j * r) * w_j) * a(z_j)), a = silu or sigmoid
 *   bwd: gw_j = g_j * w_j; s = sum_j gw_j * x_j (fp32 products, fp64 sum,
 *        same tree shape as ss); c = ((r * r) * r) * s / D;
 *        dx_j = bf16_rne(gw_j * r - x_j * c [+ gres_j])
 *   dgamma_j = sum over rows of (g_tj * x_tj) * r_t, summed per fixed chunk
 *        of rows (rmsnorm_bwd_partials_layout), then the chunk partials in a
 *        fixed order (deterministic for a given T, no atomics).
 * Batch invariance: every row's y, rstd and dx are bitwise identical whatever
 * the batch size T, the row's index, the neighbouring rows, padding rows or
 * row strides. The kernel variant and every reduction tree are chosen from D
 * alone.
 *
 * Layout. Row-major [T, D] with a row stride ld >= D (in elements), last axis
 * contiguous, D <= ld <= 2^24 (RMSN_MAX_LD) with T * ld <= 2^60, and
 * 1 <= D <= 32768 (RMSN_MAX_D) for every entry point. Each lane of a row owns
 * groups of 8 consecutive elements; every reduction tree is a function of
 * ceil(D/8) alone. When D is a multiple of 8, rows move as aligned 16-byte
 * vectors: every bf16 / fp16 base pointer and ld * 2 bytes must be multiples
 * of 16 bytes. Other D need 2-byte-aligned bases only and take any
 * ld >= D: full groups move as unaligned 16-byte accesses and the partial
 * last group of a row element by element. gamma, dgamma and the workspace
 * must be 16-byte aligned; rstd 4-byte aligned.
 *
 * Ownership and streams. Every pointer is device memory owned by the caller.
 * The library never allocates, never synchronises, never changes the
 * current device and keeps no state between calls except cached
 * per-kernel occupancy figures. All work is enqueued on `stream` (a
 * hipStream_t passed as void*; NULL = the null stream) in call order.
 * Outputs must not overlap inputs or each other; overlapping ranges are
 * rejected with RMSN_ERR_ALIASING.
 *
 * Errors. Arguments are checked on the host before anything is enqueued; on
 * any error nothing is written and nothing is launched. A launch failure
 * reports RMSN_ERR_HIP. Faults during kernel execution surface at the
 * caller's next synchronisation. No C++ exception crosses the ABI. T = 0 is
 * valid and enqueues nothing, except that a non-NULL dgamma is set to zero
 * (the empty sum). eps may be 0 (then an all-zero row gives r = +inf).
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMSN_ABI_VERSION 14
#define RMSN_MAX_D 32768
#define RMSN_MAX_LD (1 << 24)

typedef enum rmsn_status {
  RMSN_OK = 0,
  RMSN_ERR_NULL = 1,           /* a required pointer is NULL */
  RMSN_ERR_SHAPE = 2,          /* T < 0, D <= 0, ld < D or ld > RMSN_MAX_LD */
  RMSN_ERR_UNSUPPORTED_D = 3,  /* D > RMSN_MAX_D; GEMM K not a positive
                                  multiple of 32 */
  RMSN_ERR_MISALIGNED = 4,     /* a pointer or ld*2 below the alignment its
                                  operand needs (see Layout) */
  RMSN_ERR_EPS = 5,            /* eps negative or not finite */
  RMSN_ERR_ALIASING = 6,       /* an output overlaps an input or another output */
  RMSN_ERR_WORKSPACE = 7,      /* workspace NULL or smaller than required */
  RMSN_ERR_HIP = 8,            /* the HIP runtime refused a launch */
  RMSN_ERR_MODE = 9            /* unknown gate activation, rounding convention or dtype */
} rmsn_status;

/* Storage types for the _dt entry points: activations are RMSN_DTYPE_BF16
 * or RMSN_DTYPE_F16, weights any of the three. */
#define RMSN_DTYPE_BF16 0
#define RMSN_DTYPE_F16 1
#define RMSN_DTYPE_F32 2

/* Gate activations of the gated norm (RL-Kernel PR "C1: zero-centred RMSNorm
 * references and CUDA kernel" names both; silu is its default). */
#define RMSN_GATE_SILU 0     /* a(z) = z * sigmoid(z) */
#define RMSN_GATE_SIGMOID 1  /* a(z) = sigmoid(z) */

/* Rounding conventions of the gated forward (the same page: its two upstream
 * implementations round at different points; in bf16 their outputs differ by
 * more than 1e-3, with fp32 inputs they agree bitwise).
 * FP32:  out = bf16(((x * r) * w) * a(z)), every product in fp32.
 * CAST:  n = bf16(x * r), nw = bf16(n * w), out = bf16(nw * a(z)): the
 *        normalised and the weighted value are cast to the input dtype
 *        before the next multiply. */
#define RMSN_GATED_ROUND_FP32 0
#define RMSN_GATED_ROUND_CAST 1

/* RMSN_ABI_VERSION of the loaded library. */
int rmsnorm_abi_version(void);

/* A static, human-readable name for a status code. */
const char* rmsnorm_status_string(int status);

/*
 * Forward. y = bf16((x * r) * w_eff); rstd[t] = r (rstd may be NULL).
 * Megatron-LM PR "Fix the batch-invariant RMSNorm forward ...", item 1;
 * RL-Kernel "[DSv4][P1-5] rmsnorm_residual", "Implementation".
 */
rmsn_status rmsnorm_fwd(const uint16_t* x, int64_t ld_x, const float* gamma,
                        int zero_centered_gamma, float eps, int64_t T,
                        int64_t D, uint16_t* y, int64_t ld_y, float* rstd,
                        void* stream);

/*
 * Forward plus residual_out = a byte copy of x, written from the same loads
 * (RL-Kernel "[DSv4][P1-5] rmsnorm_residual", "Summary": not RMSNorm(x+res)).
 */
rmsn_status rmsnorm_residual_fwd(const uint16_t* x, int64_t ld_x,
                                 const float* gamma, int zero_centered_gamma,
                                 float eps, int64_t T, int64_t D, uint16_t* y,
                                 int64_t ld_y, uint16_t* residual_out,
                                 int64_t ld_res, float* rstd, void* stream);

/*
 * SiLU-gated forward: out = bf16(((x * r) * w_eff) * silu(z)), the weight
 * multiply in fp32 (RL-Kernel "C1: zero-centred RMSNorm references and CUDA
 * kernel", the gated-norm conventions). rstd may be NULL.
 */
rmsn_status rmsnorm_gated_fwd(const uint16_t* x, int64_t ld_x,
                              const uint16_t* z, int64_t ld_z,
                              const float* gamma, int zero_centered_gamma,
                              float eps, int64_t T, int64_t D, uint16_t* out,
                              int64_t ld_out, float* rstd, void* stream);

/*
 * Gated forward with a choice of activation (RMSN_GATE_*) and rounding
 * convention (RMSN_GATED_ROUND_*); rmsnorm_gated_fwd is the SILU / FP32
 * case. a(z) is evaluated in fp32 to about 2^-16 relative (where a(z) is a
 * normal number), so the bf16 result is within 1 ulp of the correctly
 * rounded one. rstd may be NULL. An unknown activation or rounding value
 * returns RMSN_ERR_MODE.
 */
rmsn_status rmsnorm_gated_fwd_ex(const uint16_t* x, int64_t ld_x,
                                 const uint16_t* z, int64_t ld_z,
                                 const float* gamma, int zero_centered_gamma,
                                 float eps, int64_t T, int64_t D,
                                 int activation, int rounding, uint16_t* out,
                                 int64_t ld_out, float* rstd, void* stream);

/* Bytes of workspace the backward entry points need for dgamma: chunks x
 * (D rounded up to a multiple of 8) x 4 (0 when T == 0, or D invalid).
 * Depends on T and D only. */
size_t rmsnorm_bwd_workspace_bytes(int64_t T, int64_t D);

/*
 * Layout of the dgamma partials for (T, D). The batch is cut into blocks of
 * R rows (block b = rows [b*R, min(T, (b+1)*R))), the blocks into groups of
 * S consecutive blocks (group q = blocks [q*S, (q+1)*S)), and chunk k of the
 * K chunks holds the groups k, k+K, k+2K, ... Partial row k of the
 * workspace is the sum over chunk k's rows (a fixed order: from the highest
 * row block down). R depends on D only; S and K on (T, D). Writes R, S and
 * K (each pointer may be NULL) and returns RMSN_OK, or RMSN_ERR_SHAPE /
 * RMSN_ERR_UNSUPPORTED_D without writing. K = 0 when T = 0.
 */
rmsn_status rmsnorm_bwd_partials_layout(int64_t T, int64_t D, int64_t* block_rows,
                                        int64_t* group_blocks, int64_t* chunks);

/*
 * Rows R of one block of the dgamma partials (RL-Kernel PR "[DSv4][P1-5]
 * rmsnorm_residual", "Implementation": fixed-order reductions, no split-K or
 * stream-K). R is a function of D alone: every chunk of the partials is a
 * union of whole R-row blocks, and within a block the rows are added in a
 * fixed order. Which blocks form a chunk (group_blocks S and chunks K of
 * rmsnorm_bwd_partials_layout) depends on T as well: the backward spreads
 * the batch over at most one or two workgroups per compute unit, as many as
 * the batch fills. dgamma is therefore deterministic and bitwise repeatable
 * for a given (T, D), but its rounding depends on T, and a batch split over
 * several GPUs at block boundaries does not reproduce the one-GPU dgamma
 * bits (it stays within the dgamma tolerance). The per-row outputs y, rstd
 * and dx never depend on T. Returns R, or 0 when D is outside
 * [1, RMSN_MAX_D]. A host-side query: it enqueues nothing.
 */
int rmsnorm_dgamma_chunk_rows(int64_t D);

/*
 * Backward. From the upstream gradient g, the input x and the forward's
 * saved rstd: dx = bf16(gw*r - x*c [+ g_residual]) and the fp32 weight
 * gradient dgamma (Megatron-LM PR "Fix the batch-invariant RMSNorm forward
 * and its input gradient", item 2; RL-Kernel "[DSv4][P1-5] rmsnorm_residual",
 * review comment). g_residual (may be NULL) is the gradient reaching the
 * residual copy; it is added in fp32 before dx's one rounding. dx may be
 * NULL (weight gradient only) and dgamma may be NULL (input gradient only),
 * not both; gamma is required either way. When dgamma is non-NULL the
 * caller passes a workspace of at
 * least rmsnorm_bwd_workspace_bytes(T, D) bytes, 16-byte aligned; its
 * contents on return are the per-chunk partials. Two kernels on `stream`.
 */
rmsn_status rmsnorm_bwd(const uint16_t* g, int64_t ld_g, const uint16_t* x,
                        int64_t ld_x, const float* rstd, const float* gamma,
                        int zero_centered_gamma, int64_t T, int64_t D,
                        const uint16_t* g_residual, int64_t ld_gres,
                        uint16_t* dx, int64_t ld_dx, float* dgamma,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * rmsnorm_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. It calls no allocator (no hipMalloc, no hipFree).
 * The dgamma chunk partials go to a scratch array of
 * RMSN_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * copy per GPU, from the first call on that GPU until the process ends. Every
 * (T, D) the library supports fits in it (rmsnorm_bwd_workspace_bytes never
 * exceeds it); a layout that did not would return RMSN_ERR_WORKSPACE.
 * All calls on one GPU share that GPU's array and it keeps the last call's
 * partials: calls on one stream are safe, but calls that may run at the same
 * time on one GPU (unordered streams) race on it and may return a wrong
 * dgamma. The rows kernel writes every partial the finish kernel reads, so
 * nothing needs clearing between calls. With dgamma NULL (dx only) the array
 * is not used. Arguments, results and errors otherwise as rmsnorm_bwd;
 * RMSN_ERR_HIP also when the array's address cannot be obtained on the
 * current device. Two kernels on `stream`.
 */
#define RMSN_NOALLOC_SCRATCH_BYTES (32u << 20)
rmsn_status rmsnorm_bwd_noalloc(const uint16_t* g, int64_t ld_g, const uint16_t* x,
                                int64_t ld_x, const float* rstd, const float* gamma,
                                int zero_centered_gamma, int64_t T, int64_t D,
                                const uint16_t* g_residual, int64_t ld_gres, uint16_t* dx,
                                int64_t ld_dx, float* dgamma, void* stream);

/*
 * The two stages of rmsnorm_bwd, for callers that schedule them apart.
 * rmsnorm_bwd_rows writes dx (if non-NULL) and, if workspace is non-NULL,
 * the dgamma partials: workspace[k][j] (fp32, [K][Dp], Dp = D rounded up to
 * a multiple of 8, K and the chunks from rmsnorm_bwd_partials_layout) is the
 * sum over chunk k's rows in a fixed order; columns D..Dp-1 hold zeros. rmsnorm_bwd_finish sums the
 * K partials of each column in a fixed order into dgamma[D].
 * rmsnorm_bwd(...) == rmsnorm_bwd_rows(...) then rmsnorm_bwd_finish(...).
 */
rmsn_status rmsnorm_bwd_rows(const uint16_t* g, int64_t ld_g,
                             const uint16_t* x, int64_t ld_x,
                             const float* rstd, const float* gamma,
                             int zero_centered_gamma, int64_t T, int64_t D,
                             const uint16_t* g_residual, int64_t ld_gres,
                             uint16_t* dx, int64_t ld_dx, void* workspace,
                             size_t workspace_bytes, void* stream);

rmsn_status rmsnorm_bwd_finish(const void* workspace, size_t workspace_bytes,
                               int64_t T, int64_t D, float* dgamma,
                               void* stream);

/*
 * Backward of the gated forward in the FP32 rounding convention (the pages
 * give the forward only; this is its chain rule). With n = x * r,
 * nw = n * w and a, a' the gate and its derivative at z (fp32):
 *   dz = bf16((g * nw) * a'(z))
 *   gn = g * a(z), the gradient reaching nw; then dx and dgamma are those of
 *   rmsnorm_bwd with gn in place of g:
 *   dx = bf16(gw * r - x * c), gw = gn * w, c = ((r * r) * r) * sum(gw * x) / D
 *   dgamma_j = sum over rows of (gn_tj * x_tj) * r_t (same chunked order).
 * rstd is the forward's saved inverse RMS. dx, dz and dgamma may each be
 * NULL, not all three; gamma is required. The workspace rule is
 * rmsnorm_bwd's (rmsnorm_bwd_workspace_bytes). An unknown activation
 * returns RMSN_ERR_MODE. Two kernels on `stream`.
 */
rmsn_status rmsnorm_gated_bwd(const uint16_t* g, int64_t ld_g,
                              const uint16_t* x, int64_t ld_x,
                              const uint16_t* z, int64_t ld_z,
                              const float* rstd, const float* gamma,
                              int zero_centered_gamma, int64_t T, int64_t D,
                              int activation, uint16_t* dx, int64_t ld_dx,
                              uint16_t* dz, int64_t ld_dz, float* dgamma,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * rmsnorm_fwd and rmsnorm_bwd for other storage types. act_dtype
 * (RMSN_DTYPE_BF16 or RMSN_DTYPE_F16) is the type of x, y, g, g_residual
 * and dx; weight_dtype (RMSN_DTYPE_F32, _BF16 or _F16) that of gamma. Every
 * type widens to fp32 exactly and the arithmetic is rmsnorm_fwd's /
 * rmsnorm_bwd's; the zero-centred offset is added after the cast to fp32
 * (Megatron-LM PR "Fix the batch-invariant RMSNorm forward ...", item 1).
 * fp16 results round to nearest even, subnormals kept, |v| >= 65520 to
 * infinity (RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA
 * kernel" checks fp16 beside bf16). rstd and dgamma stay fp32. gamma must be
 * 16-byte aligned whatever its type. Unknown types return RMSN_ERR_MODE;
 * everything else as rmsnorm_fwd / rmsnorm_bwd.
 */
rmsn_status rmsnorm_fwd_dt(int act_dtype, int weight_dtype, const void* x,
                           int64_t ld_x, const void* gamma,
                           int zero_centered_gamma, float eps, int64_t T,
                           int64_t D, void* y, int64_t ld_y, float* rstd,
                           void* stream);

rmsn_status rmsnorm_bwd_dt(int act_dtype, int weight_dtype, const void* g,
                           int64_t ld_g, const void* x, int64_t ld_x,
                           const float* rstd, const void* gamma,
                           int zero_centered_gamma, int64_t T, int64_t D,
                           const void* g_residual, int64_t ld_gres, void* dx,
                           int64_t ld_dx, float* dgamma, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Fused add-norm forward (RL-Kernel PR "C1: zero-centred RMSNorm references
 * and CUDA kernel", decoder-norm note: all decoder norms but the first take a
 * residual, through a fused add that normalises the fp32 sum; the page has
 * no reference arithmetic, this is its plainest reading):
 *   h = fp32(x) + fp32(residual)         (one fp32 rounding)
 *   ss = sum_j fp32(h_j * h_j)           (fp64 sum along the fixed tree)
 *   r = 1/sqrt(ss / D + eps) as in rmsnorm_fwd; rstd[t] = r (may be NULL)
 *   y = bf16((h * r) * w_eff); residual_out = bf16(h), the updated residual.
 * In place: y may be x itself and residual_out may be residual itself (the
 * same pointer and row stride); any other overlap returns
 * RMSN_ERR_ALIASING. Other errors as rmsnorm_fwd.
 */
rmsn_status rmsnorm_add_fwd(const uint16_t* x, int64_t ld_x,
                            const uint16_t* residual, int64_t ld_res,
                            const float* gamma, int zero_centered_gamma,
                            float eps, int64_t T, int64_t D, uint16_t* y,
                            int64_t ld_y, uint16_t* residual_out,
                            int64_t ld_rout, float* rstd, void* stream);

/*
 * Backward of rmsnorm_add_fwd from the forward's saved rstd. h = x + residual
 * is recomputed exactly as in the forward; with gw = g * w_eff,
 * s = sum_j gw_j * h_j (fp32 products, fp64 sum), c = ((r*r)*r) * s / D:
 *   dh = bf16(gw * r - h * c [+ g_residual_out])
 * dh is the gradient of both x and residual (d h / d x = d h / d residual =
 * 1); g_residual_out (may be NULL) is the gradient arriving at residual_out,
 * added in fp32 before the one rounding. dgamma_j = sum over rows of
 * (g_tj * h_tj) * r_t, chunked as rmsnorm_bwd's. dh or dgamma may be NULL,
 * not both; gamma is required; the workspace rule is rmsnorm_bwd's. No
 * output may overlap an input. Two kernels on `stream`.
 */
rmsn_status rmsnorm_add_bwd(const uint16_t* g, int64_t ld_g,
                            const uint16_t* x, int64_t ld_x,
                            const uint16_t* residual, int64_t ld_res,
                            const float* rstd, const float* gamma,
                            int zero_centered_gamma, int64_t T, int64_t D,
                            const uint16_t* g_residual_out, int64_t ld_gro,
                            uint16_t* dh, int64_t ld_dh, float* dgamma,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* The first stage of rmsnorm_add_bwd alone: dh (if non-NULL) and, if
 * workspace is non-NULL, the dgamma partials that rmsnorm_bwd_finish turns
 * into dgamma. */
rmsn_status rmsnorm_add_bwd_rows(const uint16_t* g, int64_t ld_g,
                                 const uint16_t* x, int64_t ld_x,
                                 const uint16_t* residual, int64_t ld_res,
                                 const float* rstd, const float* gamma,
                                 int zero_centered_gamma, int64_t T, int64_t D,
                                 const uint16_t* g_residual_out, int64_t ld_gro,
                                 uint16_t* dh, int64_t ld_dh, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * The gated norm and the fused add-norm for other storage types, as
 * rmsnorm_fwd_dt / rmsnorm_bwd_dt are for the plain norm. act_dtype
 * (RMSN_DTYPE_BF16 or RMSN_DTYPE_F16) is the type of every activation
 * operand: x, z, residual, g, g_residual_out and the outputs out, y,
 * residual_out, dx, dz and dh; weight_dtype (RMSN_DTYPE_F32, _BF16 or _F16)
 * that of gamma. Each widens to fp32 exactly and the arithmetic is that of
 * rmsnorm_gated_fwd_ex, rmsnorm_gated_bwd, rmsnorm_add_fwd and
 * rmsnorm_add_bwd, with every rounding of a result to bf16 there made to
 * act_dtype here (fp16: nearest even, subnormals kept, overflow to
 * infinity). That includes the two intermediate casts of the gated
 * RMSN_GATED_ROUND_CAST convention, which round to the input dtype
 * (RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel",
 * gated-norm conventions; its contract checks fp16 beside bf16). In the
 * fused add, h = fp32(x) + fp32(residual) and residual_out = act_dtype(h).
 * rstd and dgamma stay fp32; gamma must be 16-byte aligned whatever its
 * type. Unknown types return RMSN_ERR_MODE; arguments, aliasing rules,
 * workspace and errors otherwise as the bf16 entry points named above.
 */
rmsn_status rmsnorm_gated_fwd_dt(int act_dtype, int weight_dtype, const void* x,
                                 int64_t ld_x, const void* z, int64_t ld_z,
                                 const void* gamma, int zero_centered_gamma,
                                 float eps, int64_t T, int64_t D, int activation,
                                 int rounding, void* out, int64_t ld_out,
                                 float* rstd, void* stream);

rmsn_status rmsnorm_gated_bwd_dt(int act_dtype, int weight_dtype, const void* g,
                                 int64_t ld_g, const void* x, int64_t ld_x,
                                 const void* z, int64_t ld_z, const float* rstd,
                                 const void* gamma, int zero_centered_gamma,
                                 int64_t T, int64_t D, int activation, void* dx,
                                 int64_t ld_dx, void* dz, int64_t ld_dz,
                                 float* dgamma, void* workspace,
                                 size_t workspace_bytes, void* stream);

rmsn_status rmsnorm_add_fwd_dt(int act_dtype, int weight_dtype, const void* x,
                               int64_t ld_x, const void* residual, int64_t ld_res,
                               const void* gamma, int zero_centered_gamma,
                               float eps, int64_t T, int64_t D, void* y,
                               int64_t ld_y, void* residual_out, int64_t ld_rout,
                               float* rstd, void* stream);

rmsn_status rmsnorm_add_bwd_dt(int act_dtype, int weight_dtype, const void* g,
                               int64_t ld_g, const void* x, int64_t ld_x,
                               const void* residual, int64_t ld_res,
                               const float* rstd, const void* gamma,
                               int zero_centered_gamma, int64_t T, int64_t D,
                               const void* g_residual_out, int64_t ld_gro,
                               void* dh, int64_t ld_dh, float* dgamma,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Batch-invariant BF16 GEMM, Y = X @ W.T (TransformerEngine issue "Expose
 * Batch Invariant Kernels", point 3: the library GEMM chose its algorithm,
 * and so its reduction order, from the whole shape; fixed tiles and a fixed
 * K loop make a row of Y independent of the other rows and of M).
 * X bf16 [M, K] and W bf16 [N, K], row-major with K contiguous; Y bf16
 * [M, N] row-major. Each output is a dot product accumulated in fp32 from
 * zero over K in ascending steps of 16 (one 32x32x16 bf16 matrix-core step
 * each; no split-K) and rounded once to bf16. The output tile a workgroup
 * computes follows M and N (bigemm_bf16_tile), but an output's arithmetic
 * does not, so every row of Y is bitwise identical whatever M, the row's
 * position and the other rows are.
 * Supported: K a positive multiple of 32; K <= ld_x, ld_w <= 2^21 and
 * ld_x, ld_w multiples of 8 with X and W 16-byte aligned; N <= ld_y <=
 * 2^60 / M, Y 2-byte aligned. Errors: RMSN_ERR_SHAPE (negative sizes,
 * strides out of range, or more than 2^31 - 1 tiles of 32 x 64), RMSN_ERR_UNSUPPORTED_D (K not a positive
 * multiple of 32), RMSN_ERR_NULL, RMSN_ERR_MISALIGNED, RMSN_ERR_ALIASING
 * (Y overlaps X or W), RMSN_ERR_HIP.
 * M = 0 or N = 0 enqueue nothing. No workspace; one kernel on `stream`.
 */
rmsn_status bigemm_bf16_xwt(const uint16_t* x, int64_t ld_x, const uint16_t* w,
                            int64_t ld_w, int64_t M, int64_t N, int64_t K,
                            uint16_t* y, int64_t ld_y, void* stream);

/* The output tile (rows of Y x columns of Y per workgroup) bigemm_bf16_xwt
 * uses for an M x N product: of 256x256, 128x256, 128x128, 64x128 and
 * 32x64, the one with the least estimated time, ceil(tiles / 256) rounds
 * (one tile per compute unit) times that tile's measured time per round
 * (113.8, 64.0, 39.6, 25.8 and 19.4 us at K = 4096); ties go to the larger
 * tile. The choice depends on M and N only. A host-side query: it enqueues
 * nothing and needs no GPU.
 * Errors: RMSN_ERR_SHAPE (M or N negative), RMSN_ERR_NULL (an output
 * pointer is NULL). */
rmsn_status bigemm_bf16_tile(int64_t M, int64_t N, int64_t* tile_m, int64_t* tile_n);

#ifdef __cplusplus
}
#endif
#endif /* RMSNORM_MI355X_H */
