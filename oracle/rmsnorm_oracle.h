/*
 * CPU oracle for batch-invariant RMSNorm — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct host implementation of what the GPU
 * library computes, used to check it. Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load or call this library; the
 * GPU library never links, includes or calls it, and the two share no code.
 *
 * Sources (pages by title; section / equation named, no line numbers):
 *  [MEG]  Megatron-LM PR "Fix the batch-invariant RMSNorm forward and its
 *         input gradient", section "What does this PR do?": item 1 (the
 *         zero-centred offset is added after the cast to fp32, in forward and
 *         backward alike) and item 2 (the input-gradient equation, the weight
 *         entering once per term; the weight gradient as the plain sum).
 *  [C1]   RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel":
 *         the +1 of the zero-centred weight is an fp32 operation; the gated
 *         norm's SiLU gate with the weight multiply in fp32; the backward
 *         reuses the forward's saved rstd.
 *  [TE]   TransformerEngine issue "Expose Batch Invariant Kernels": the
 *         batch-invariant BF16 GEMM Y = X @ W.T (point 3).
 *  [RES]  RL-Kernel PR "[DSv4][P1-5] rmsnorm_residual", sections "Summary",
 *         "Implementation" and the review comment: output is RMSNorm(x) plus
 *         a byte copy of x; bf16 activations, fp32 gamma, fp32 saved inverse
 *         RMS, fp32 dgamma; r = rsqrt(mean(x^2) + eps); y = (x * r) * gamma;
 *         mul and add rounded separately; dx gains the residual branch's
 *         gradient; dgamma = sum over tokens of dy * x * r.
 *
 * Arithmetic modes (argument `mode`):
 *  ORACLE_R64 (0, the parity reference): every elementwise step is one fp32
 *     operation rounded to nearest-even, with no FMA contraction (built with
 *     -ffp-contract=off). The three reductions (sum of squares, the row dot
 *     product, dgamma over rows) add the fp32 terms in ascending index order
 *     in double and round the total to fp32 once, so their result does not
 *     depend on any reduction tree. rsqrt is 1/sqrt taken in double and
 *     rounded to fp32.
 *  ORACLE_A32 (1): identical, except the three reductions accumulate in fp32
 *     in ascending order (the "ascending FP32 reductions" of [RES]). Used only
 *     to report how far that convention sits from R64.
 *  The *_f64 entry points take double inputs and compute everything in
 *     double with no intermediate rounding; they are the exact formulas used
 *     for finite-difference and invariant checks.
 *
 * Layouts: activations are row-major [T, D] with row stride ld >= D
 * elements; bf16 values travel as raw uint16_t bits. gamma, rstd and dgamma
 * are fp32. All pointers are host memory owned by the caller. Functions
 * return 0 on success and -1 on a bad argument (NULL where an array is
 * needed, T < 0, D <= 0, ld < D), writing nothing in that case.
 */
#ifndef RMSNORM_ORACLE_H
#define RMSNORM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_R64 = 0, ORACLE_A32 = 1 };

/* bf16 codec: decode is exact (bits << 16); encode rounds to nearest,
 * ties to even, keeps subnormals, sends overflow to +-inf and maps NaN to a
 * quiet NaN of the same sign. */
void oracle_bf16_decode(const uint16_t* in, int64_t n, float* out);
void oracle_bf16_encode(const float* in, int64_t n, uint16_t* out);

/* w_eff[j] = gamma[j], plus 1.0f in fp32 when zero_centered ([MEG] item 1). */
int oracle_weights(const float* gamma, int zero_centered, int64_t D, float* w_eff);

/* Forward: rstd[t] = rsqrt(mean_j x^2 + eps); y = bf16((x * r) * w_eff).
 * rstd may be NULL. */
int oracle_rmsnorm_fwd(int mode, const uint16_t* x, int64_t ld_x,
                       const float* gamma, int zero_centered, float eps,
                       int64_t T, int64_t D, uint16_t* y, int64_t ld_y,
                       float* rstd);

/* Forward plus residual_out = a byte copy of x ([RES] "Summary"). */
int oracle_rmsnorm_residual_fwd(int mode, const uint16_t* x, int64_t ld_x,
                                const float* gamma, int zero_centered,
                                float eps, int64_t T, int64_t D, uint16_t* y,
                                int64_t ld_y, uint16_t* residual_out,
                                int64_t ld_res, float* rstd);

/* SiLU-gated forward ([C1]): n = (x * r) * w_eff in fp32, silu(z) =
 * z / (1 + exp(-z)) evaluated in double and rounded to fp32,
 * out = bf16(n * silu(z)). rstd may be NULL. */
int oracle_rmsnorm_gated_fwd(int mode, const uint16_t* x, int64_t ld_x,
                             const uint16_t* z, int64_t ld_z,
                             const float* gamma, int zero_centered, float eps,
                             int64_t T, int64_t D, uint16_t* out,
                             int64_t ld_out, float* rstd);

/* Input gradient from the saved rstd ([MEG] item 2, [RES] review):
 *   gw = g * w_eff; s = sum_j gw_j * x_j; c = ((r*r)*r)*s / D;
 *   dx = bf16((gw * r - x * c) [+ gres]).
 * gres may be NULL (ld_gres ignored then). */
int oracle_rmsnorm_bwd_dx(int mode, const uint16_t* g, int64_t ld_g,
                          const uint16_t* x, int64_t ld_x, const float* rstd,
                          const float* gamma, int zero_centered, int64_t T,
                          int64_t D, const uint16_t* gres, int64_t ld_gres,
                          uint16_t* dx, int64_t ld_dx);

/* Weight gradient over `ncols` columns: dgamma[j] = sum over t ascending of
 * (g[t][j] * x[t][j]) * rstd[t]. Independent of the zero-centred flag since
 * d(w_eff)/d(gamma) = 1. T = 0 gives zeros. */
int oracle_rmsnorm_dgamma(int mode, const uint16_t* g, int64_t ld_g,
                          const uint16_t* x, int64_t ld_x, const float* rstd,
                          int64_t T, int64_t ncols, float* dgamma);

/* Exact (double) forms. w_eff = gamma (+1.0 when zero_centered). */
int oracle_rmsnorm_fwd_f64(const double* x, const double* gamma,
                           int zero_centered, double eps, int64_t T, int64_t D,
                           double* y, double* rstd);
int oracle_rmsnorm_gated_fwd_f64(const double* x, const double* z,
                                 const double* gamma, int zero_centered,
                                 double eps, int64_t T, int64_t D, double* out);
/* dx (may be NULL) and dgamma (may be NULL) of L = sum g*y, with r recomputed
 * in double from x. gres (may be NULL) is added to dx. */
int oracle_rmsnorm_bwd_f64(const double* g, const double* x,
                           const double* gamma, int zero_centered, double eps,
                           int64_t T, int64_t D, const double* gres,
                           double* dx, double* dgamma);

/* ---- Gated-norm variants -------------------------------------------------
 * activation: ORACLE_GATE_SILU a(z) = z*sigmoid(z), ORACLE_GATE_SIGMOID
 * a(z) = sigmoid(z) (the two gate activations [C1] names).
 * convention: ORACLE_GATED_FP32 (the weight multiply in fp32, one rounding
 * at the end: out = bf16(fp32(fp32(x*r)*w) * a(z))) or ORACLE_GATED_CAST
 * (the other upstream's convention as read here: the normalised value and
 * the weighted value are each cast to the input dtype before the next
 * multiply, out = bf16(fp32(bf16(fp32(bf16(x*r)*w)) * a(z))). With fp32
 * inputs those casts are no-ops and the two conventions agree bitwise.)
 * a(z) is evaluated in double and rounded to fp32.
 */
enum { ORACLE_GATE_SILU = 0, ORACLE_GATE_SIGMOID = 1 };
enum { ORACLE_GATED_FP32 = 0, ORACLE_GATED_CAST = 1 };

int oracle_rmsnorm_gated_fwd_ex(int mode, int activation, int convention,
                                const uint16_t* x, int64_t ld_x,
                                const uint16_t* z, int64_t ld_z,
                                const float* gamma, int zero_centered,
                                float eps, int64_t T, int64_t D,
                                uint16_t* out, int64_t ld_out, float* rstd);

/* The same forward on fp32 inputs and outputs (contiguous [T, D]): every
 * cast to the input dtype is then the identity. */
int oracle_rmsnorm_gated_fwd_f32io(int activation, int convention,
                                   const float* x, const float* z,
                                   const float* gamma, int zero_centered,
                                   float eps, int64_t T, int64_t D, float* out);

/* Gated backward (the fp32 convention), from the saved rstd. With
 * n = fp32(x*r), nw = fp32(n*w), a = fp32(a(z)), a' = fp32(a'(z)) (double,
 * rounded), and g the gradient of out:
 *   dz = bf16(fp32(fp32(g*nw) * a'))
 *   gn = fp32(g*a)                      (gradient reaching nw)
 *   dx = the plain input gradient with gn in place of g:
 *        gw = fp32(gn*w); s = sum gw*x; c = ((r*r)*r)*s/D;
 *        dx = bf16(fp32(gw*r) - fp32(x*c))
 * dx or dz may be NULL. */
int oracle_rmsnorm_gated_bwd(int mode, int activation, const uint16_t* g,
                             int64_t ld_g, const uint16_t* x, int64_t ld_x,
                             const uint16_t* z, int64_t ld_z, const float* rstd,
                             const float* gamma, int zero_centered, int64_t T,
                             int64_t D, uint16_t* dx, int64_t ld_dx,
                             uint16_t* dz, int64_t ld_dz);

/* dgamma[j] = sum over t ascending of fp32(fp32(gn[t][j]*x[t][j]) * r[t]),
 * gn = fp32(g*a(z)), over `ncols` columns. */
int oracle_rmsnorm_gated_dgamma(int mode, int activation, const uint16_t* g,
                                int64_t ld_g, const uint16_t* x, int64_t ld_x,
                                const uint16_t* z, int64_t ld_z,
                                const float* rstd, int64_t T, int64_t ncols,
                                float* dgamma);

/* Exact forms of the gated forward and backward (contiguous [T, D]). */
int oracle_rmsnorm_gated_fwd_ex_f64(int activation, const double* x,
                                    const double* z, const double* gamma,
                                    int zero_centered, double eps, int64_t T,
                                    int64_t D, double* out);
int oracle_rmsnorm_gated_bwd_f64(int activation, const double* g,
                                 const double* x, const double* z,
                                 const double* gamma, int zero_centered,
                                 double eps, int64_t T, int64_t D, double* dx,
                                 double* dz, double* dgamma);

/* ---- Fused add-RMSNorm -------------------------------------------------
 * The residual form of the decoder norm ([C1]: fused_add_rms_norm
 * "normalises the fp32 sum"; the page has no reference arithmetic for it,
 * so this is the plainest reading):
 *   h = fp32(x) + fp32(residual)          (one fp32 rounding)
 *   ss = sum_j fp32(h_j * h_j)            (ascending; double in R64)
 *   r = rsqrt(fp32(ss / D) + eps); y = bf16((h * r) * w_eff);
 *   residual_out = bf16(h); rstd[t] = r (rstd may be NULL).
 * Backward, h recomputed from x and residual exactly as above:
 *   gw = g * w_eff; s = sum gw * h; c = ((r*r)*r)*s / D;
 *   dh = bf16((gw * r - h * c) [+ g_rout])
 * dh is the gradient of both x and residual; g_rout (may be NULL) is the
 * gradient arriving at residual_out. dgamma[j] = sum over t ascending of
 * fp32(fp32(g*h) * r). dh or dgamma may be NULL, not both. */
int oracle_rmsnorm_add_fwd(int mode, const uint16_t* x, int64_t ld_x,
                           const uint16_t* residual, int64_t ld_res,
                           const float* gamma, int zero_centered, float eps,
                           int64_t T, int64_t D, uint16_t* y, int64_t ld_y,
                           uint16_t* residual_out, int64_t ld_rout, float* rstd);
int oracle_rmsnorm_add_bwd(int mode, const uint16_t* g, int64_t ld_g,
                           const uint16_t* x, int64_t ld_x,
                           const uint16_t* residual, int64_t ld_res,
                           const float* rstd, const float* gamma,
                           int zero_centered, int64_t T, int64_t D,
                           const uint16_t* g_rout, int64_t ld_gro, uint16_t* dh,
                           int64_t ld_dh, float* dgamma);
/* Exact forms (contiguous [T, D]): h = x + residual in double; h_out and
 * rstd may be NULL; dh is the gradient of L = sum g*y + sum g_rout*h with
 * respect to h (g_rout may be NULL). */
int oracle_rmsnorm_add_fwd_f64(const double* x, const double* residual,
                               const double* gamma, int zero_centered, double eps,
                               int64_t T, int64_t D, double* y, double* h_out,
                               double* rstd);
int oracle_rmsnorm_add_bwd_f64(const double* g, const double* x,
                               const double* residual, const double* gamma,
                               int zero_centered, double eps, int64_t T,
                               int64_t D, const double* g_rout, double* dh,
                               double* dgamma);

/* ---- Activation and weight dtypes --------------------------------------
 * Storage types: activations (x, g, gres, y, dx) ORACLE_BF16 or ORACLE_F16,
 * weights ORACLE_F32, ORACLE_BF16 or ORACLE_F16 (gamma points at that type).
 * Each widens to fp32 exactly; the weight offset (+1.0f) follows the cast
 * ([MEG] item 1). Results round to the activation type (RNE; binary16:
 * subnormals kept, |v| >= 65520 -> inf). The arithmetic is that of
 * oracle_rmsnorm_fwd / _bwd_dx / _dgamma (squares and g*x of fp16 inputs
 * are exact in fp32 too), which equal the _dt forms with (BF16, F32). */
enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_F32 = 2 };
void oracle_f16_decode(const uint16_t* in, int64_t n, float* out);
void oracle_f16_encode(const float* in, int64_t n, uint16_t* out);
int oracle_rmsnorm_fwd_dt(int mode, int act_dtype, int weight_dtype,
                          const uint16_t* x, int64_t ld_x, const void* gamma,
                          int zero_centered, float eps, int64_t T, int64_t D,
                          uint16_t* y, int64_t ld_y, float* rstd);
int oracle_rmsnorm_bwd_dx_dt(int mode, int act_dtype, int weight_dtype,
                             const uint16_t* g, int64_t ld_g, const uint16_t* x,
                             int64_t ld_x, const float* rstd, const void* gamma,
                             int zero_centered, int64_t T, int64_t D,
                             const uint16_t* gres, int64_t ld_gres, uint16_t* dx,
                             int64_t ld_dx);
int oracle_rmsnorm_dgamma_dt(int mode, int act_dtype, const uint16_t* g,
                             int64_t ld_g, const uint16_t* x, int64_t ld_x,
                             const float* rstd, int64_t T, int64_t ncols,
                             float* dgamma);

/* The gated norm and the fused add-norm in other storage types: the same
 * definitions as oracle_rmsnorm_gated_fwd_ex / _gated_bwd / _gated_dgamma and
 * oracle_rmsnorm_add_fwd / _add_bwd, with activations ORACLE_BF16 or
 * ORACLE_F16 and weights ORACLE_F32, ORACLE_BF16 or ORACLE_F16 (gamma points at
 * that type). The gated cast convention rounds to the activations' type. With
 * (ORACLE_BF16, ORACLE_F32) they equal those functions bitwise. */
int oracle_rmsnorm_gated_fwd_dt(int mode, int act_dtype, int weight_dtype, int activation,
                                int convention, const uint16_t* x, int64_t ld_x,
                                const uint16_t* z, int64_t ld_z, const void* gamma,
                                int zero_centered, float eps, int64_t T, int64_t D, uint16_t* out,
                                int64_t ld_out, float* rstd);
int oracle_rmsnorm_gated_bwd_dt(int mode, int act_dtype, int weight_dtype, int activation,
                                const uint16_t* g, int64_t ld_g, const uint16_t* x, int64_t ld_x,
                                const uint16_t* z, int64_t ld_z, const float* rstd,
                                const void* gamma, int zero_centered, int64_t T, int64_t D,
                                uint16_t* dx, int64_t ld_dx, uint16_t* dz, int64_t ld_dz);
int oracle_rmsnorm_gated_dgamma_dt(int mode, int act_dtype, int activation, const uint16_t* g,
                                   int64_t ld_g, const uint16_t* x, int64_t ld_x,
                                   const uint16_t* z, int64_t ld_z, const float* rstd, int64_t T,
                                   int64_t ncols, float* dgamma);
int oracle_rmsnorm_add_fwd_dt(int mode, int act_dtype, int weight_dtype, const uint16_t* x,
                              int64_t ld_x, const uint16_t* residual, int64_t ld_res,
                              const void* gamma, int zero_centered, float eps, int64_t T, int64_t D,
                              uint16_t* y, int64_t ld_y, uint16_t* residual_out, int64_t ld_rout,
                              float* rstd);
int oracle_rmsnorm_add_bwd_dt(int mode, int act_dtype, int weight_dtype, const uint16_t* g,
                              int64_t ld_g, const uint16_t* x, int64_t ld_x,
                              const uint16_t* residual, int64_t ld_res, const float* rstd,
                              const void* gamma, int zero_centered, int64_t T, int64_t D,
                              const uint16_t* g_rout, int64_t ld_gro, uint16_t* dh, int64_t ld_dh,
                              float* dgamma);

/* ---- Batch-invariant GEMM ([TE] point 3: BF16 Y = X @ W.T) -------------
 * X bf16 [M, K] (row stride ldx), W bf16 [N, K] (ldw), Y bf16 [M, N] (ldy):
 * Y[i][j] = bf16(fp32(sum over k ascending of X[i][k] * W[j][k])), the sum in
 * double. Y_exact (may be NULL, contiguous [M, N]) receives the double sums. */
int oracle_gemm_xwt(const uint16_t* X, int64_t ldx, const uint16_t* W,
                    int64_t ldw, int64_t M, int64_t N, int64_t K, uint16_t* Y,
                    int64_t ldy, double* Y_exact);

/* Test-only defect planting, so the tests can show that their checks catch
 * the two defects [MEG] fixes: 0 = none; 1 = the forward ignores the
 * zero-centred offset (the backward still honours it); 2 = the second term
 * of dx is multiplied by w_eff[k] a second time. Affects R64/A32 and f64. */
void oracle_set_mutation(int mutation);

#ifdef __cplusplus
}
#endif
#endif
