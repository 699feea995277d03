/*
 * ln_oracle.h -- float64 CPU oracle for fused LayerNorm forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this code: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can check the GPU library against a plain,
 * slow, obviously correct definition.  It shares no source with the GPU
 * library (no headers, helpers, constants or tables).
 *
 * Sources ("the pages"):
 *   [L10]  "Accelerating Transformer on GPU (I): Kernel Fusion and LightSeq
 *          Inference" (CMU 11-868 lecture-10 notes)
 *   [L11]  "Accelerating Transformer on GPU (II): Training with LightSeq2"
 *          (CMU 11-868 lecture-11 notes)
 *   [FP]   "GPU Performance from First Principles" (CS349D prerequisite P1)
 *   [BLOG] "AI infra 学习记录(2): 从 LayerNorm 算子熟悉常见的算子优化方法"
 *   [LLMC] "02 · llmc/ 的 CUDA kernel 层" (llm.c CUDA kernel walk-through)
 *
 * Conventions: every tensor is row-major [rows, m], contiguous, held as
 * double.  Inputs that the GPU reads in a storage type (fp32/fp16/bf16) are
 * passed here as the exact double value of the stored number; mean and rstd,
 * when they are inputs, are the exact double value of the stored fp32.
 * All arithmetic is float64 unless a function says it emulates fp32.
 *
 * Pins: every function is checked in tests/test_oracle_pins.py against
 * something other than itself (worked examples printed on the pages, closed
 * forms, identities, finite differences); the Philox4x32-10 round function,
 * for which the pages print no known-answer values, is pinned against an
 * independent implementation of the published generator (rocRAND's host
 * engine) in tests/test_philox_pin.py.
 */
#ifndef MBROW_LN_ORACLE_H
#define MBROW_LN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats the oracle can round to. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* Round a double to the nearest value of the storage format, ties to even,
 * overflow to +-inf, NaN stays NaN; returns that value as a double.
 * [FP] §7.1-7.3 (bf16 = 8 significant bits, fp16 = 11, spacing grows with
 * magnitude) and exercise 6 (1001 -> 1000, 257 -> 256 tie to even). */
double orc_round(double v, int fmt);
void orc_round_array(const double* in, double* out, int64_t n, int fmt);

/* LayerNorm forward by its definition, two passes per row.
 * [L11] §2.1: xhat = (x - mu)/sigma, sigma = sqrt(var + eps),
 * y = gamma*xhat + beta, save mu and r = 1/sigma per row.
 * [L10] §4.2: var = mean((x - mu)^2) (population variance, divide by m).
 * Any of y, mean, rstd may be NULL. */
void orc_ln_fwd(const double* x, const double* gamma, const double* beta,
                int64_t rows, int64_t m, double eps,
                double* y, double* mean, double* rstd);

/* Row mean and population variance by Welford's one-element update over each
 * half of the row, then one Chan merge of the two halves.
 * [L10] §4.2 (per-thread (count, mean, M2), pairwise merge formula). */
void orc_row_stats_welford(const double* x, int64_t rows, int64_t m,
                           double* mean, double* var);

/* fp32 emulations used to show the variance hazard of [L10] §4.2.
 * naive: sum and sum of squares accumulated in float, var = E[x^2] - E[x]^2.
 * chan:  'lanes' strided per-lane Welford states in float, merged pairwise
 *        (lane i with lane i + lanes/2, ...) with the Chan formula in float;
 *        lanes must be a power of two. */
void orc_var_naive_f32(const double* x, int64_t rows, int64_t m, double* var);
void orc_var_chan_f32(const double* x, int64_t rows, int64_t m, int lanes,
                      double* var);

/* Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11): counter ctr[4], key key[2] -> out[4]. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                       uint32_t out[4]);

/* Dropout keep threshold for probability p: floor(p * 65536 + 0.5),
 * computed in double from the float p.  An element is kept iff its 16-bit
 * uniform u satisfies u >= threshold. */
uint32_t orc_dropout_threshold(float p);

/* Keep mask for a [rows, m] tensor (1 = kept).  The pages fix only that the
 * mask is regenerated from a stored seed ([L11] §3.3) and drawn per element
 * by the fused kernel ([L10] §5.1); the function of (seed, row, col) is this
 * library's own: key = (seed low 32, seed high 32); counter = (col >> 3,
 * row low 32, row high 32, 0); column col takes the 16-bit half
 * (col & 1) of output word (col & 7) >> 1. */
void orc_dropout_keep(uint64_t seed, float p, int64_t rows, int64_t m,
                      uint8_t* keep);
/* The same mask for rows [row0, row0 + rows) of a tensor (keep holds
 * rows x m entries): for checking sampled rows of very large tensors. */
void orc_dropout_keep_rows(uint64_t seed, float p, int64_t row0, int64_t rows, int64_t m,
                           uint8_t* keep);

/* Bias + dropout + residual, [L10] §2.3 (bias add, dropout, then residual):
 * t = x + bias; d = keep ? t / (1 - p) : 0; z = residual + d.  Exact in
 * double; z is NOT rounded (round it with orc_round_array). */
void orc_bias_dropout_residual(const double* x, const double* bias,
                               const double* residual, const uint8_t* keep,
                               float p, int64_t rows, int64_t m, double* z);

/* Backward of the bias + dropout + residual prologue ([L10] §2.3 order: bias
 * add, dropout, residual add; [L11] §3.3: the mask is regenerated from the
 * seed instead of stored).  With z = residual + keep * (x + bias) / (1 - p)
 * and dz the gradient reaching z (the LayerNorm's dx plus any gradient from
 * z's other uses), by the chain rule:
 *   dresidual = dz (the caller keeps dz);
 *   dx_j = keep_j ? dz_j / (1 - p) : 0;
 *   dbias_j = sum over rows of dx_rj (row order); sbias_j = sum of |dx_rj|
 * (sbias may be NULL). */
void orc_dropout_residual_bwd(const double* dz, const uint8_t* keep, float p,
                              int64_t rows, int64_t m, double* dx,
                              double* dbias, double* sbias);

/* LayerNorm backward dx, the x-hat form ([L11] §2.1, "HW4" form):
 * g = gamma*dy, xhat = (x - mu)*r, A = sum g, B = sum g*xhat,
 * dx = r * (g - (A + xhat*B)/m). */
void orc_ln_bwd_dx_hw4(const double* dy, const double* x, const double* gamma,
                       const double* mean, const double* rstd,
                       int64_t rows, int64_t m, double* dx);

/* Magnitude of the terms that form each dx_j in the x-hat form:
 * scale_j = r * (|g_j| + (sum_k |g_k| + |xhat_j| * sum_k |g_k xhat_k|) / m).
 * A float32 evaluation of dx_j rounds quantities of at most this size, so its
 * error is bounded by a small multiple of 2^-24 * scale_j (used by the
 * tolerance rule, not by the result). */
void orc_ln_bwd_dx_scale(const double* dy, const double* x, const double* gamma,
                         const double* mean, const double* rstd,
                         int64_t rows, int64_t m, double* scale);

/* LayerNorm backward dx, the slides form ([L11] §2.1):
 * dx = g/sigma + alpha*sum g + beta*sum g*x with
 * alpha = ((x - mu)*mu - sigma^2)/(m sigma^3), beta = (mu - x)/(m sigma^3),
 * sigma = 1/r. */
void orc_ln_bwd_dx_slides(const double* dy, const double* x,
                          const double* gamma, const double* mean,
                          const double* rstd, int64_t rows, int64_t m,
                          double* dx);

/* Column gradients ([L11] §2.1 and §2.4): dgamma_j = sum_rows dy*xhat,
 * dbeta_j = sum_rows dy, summed in row order.  Also the sums of absolute
 * terms sgamma_j = sum |dy*xhat|, sbeta_j = sum |dy| (for error bounds).
 * sgamma / sbeta may be NULL. */
void orc_ln_bwd_params(const double* dy, const double* x, const double* mean,
                       const double* rstd, int64_t rows, int64_t m,
                       double* dgamma, double* dbeta,
                       double* sgamma, double* sbeta);

/* RMSNorm ([FP] §6, "fused add + RMSNorm": one sum of squares, no mean):
 *   rstd = 1 / sqrt((1/m) sum_j x_j^2 + eps);  y_j = gamma_j * x_j * rstd.
 * The fused kernel adds the residual first and normalises the stored sum;
 * that add is done by the caller here. */
void orc_rmsnorm_fwd(const double* x, const double* gamma, int64_t rows, int64_t m,
                     double eps, double* y, double* rstd);

/* RMSNorm backward, the chain rule of the above with xhat = x * rstd and
 * g = gamma * dy:  dx_j = rstd * (g_j - xhat_j * (sum_k g_k xhat_k) / m);
 * dgamma_j = sum over rows of dy * xhat (row order), sgamma_j = sum of
 * |dy * xhat| (may be NULL).  rstd is the saved float32 value. */
void orc_rmsnorm_bwd(const double* dy, const double* x, const double* gamma,
                     const double* rstd, int64_t rows, int64_t m, double* dx,
                     double* dgamma, double* sgamma);

/* Attention softmax forward ([L10] §4.1: per row, scale, add the mask, the
 * row maximum, exp of the difference, the row sum, divide), one row at a
 * time in double:
 *   t_j = scale * x_j + (mask ? mask[(r / rows_per_mask) * m + j] : 0);
 *   causal: t_j = -inf for keys j > q, q = r mod m (square score blocks);
 *   mx = max_j t_j; y_j = exp(t_j - mx) / sum_k exp(t_k - mx).
 * A row whose every key is masked (mx = -inf) gives y = 0. */
void orc_attn_softmax_fwd(const double* x, const double* mask, int64_t rows_per_mask,
                          int64_t rows, int64_t m, double scale, int causal, double* y);

/* Attention softmax backward fused with the dropout backward ([L11] §3: the
 * Jacobian y_i (delta_ij - y_j) times a vector needs one dot product; the
 * dropout backward is applied first, in registers):
 *   g_j = keep ? (keep_j ? dy_j / (1 - p) : 0) : dy_j;   s = sum_j g_j y_j;
 *   dx_j = scale * y_j * (g_j - s).
 * keep may be NULL (no dropout). */
void orc_attn_softmax_bwd(const double* dy, const double* y, const uint8_t* keep, float p,
                          int64_t rows, int64_t m, double scale, double* dx);

/* Cross-entropy of a row of logits against a class label, with label
 * smoothing, and its gradient, by the definitions ([L10] §5.2; [LLMC] §6.1
 * for the fusion of loss and gradient over a vocabulary-wide row):
 *   q = softmax(x) (computed with the row maximum subtracted),
 *   p_j = (1 - alpha) [j == label] + alpha / V,
 *   loss = -sum_j p_j log q_j,   dx_j = scale * (q_j - p_j).
 * A negative label marks an ignored row: loss 0 and dx 0.  A label >= V has
 * no target distribution: loss and dx are NaN.  x is [rows, V]; loss is
 * [rows]; dx [rows, V] may be NULL. */
void orc_cross_entropy(const double* x, const int64_t* labels, int64_t rows, int64_t V,
                       double alpha, double scale, double* loss, double* dx);

#ifdef __cplusplus
}
#endif

#endif
