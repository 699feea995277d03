/*
 * mbrow_ln.h -- C ABI of the fused LayerNorm library for AMD MI355X (gfx950).
 *
 * Sources ("the pages"):
 *   [L10]  "Accelerating Transformer on GPU (I): Kernel Fusion and LightSeq
 *          Inference" (CMU 11-868 lecture-10 notes)
 *   [L11]  "Accelerating Transformer on GPU (II): Training with LightSeq2"
 *          (CMU 11-868 lecture-11 notes)
 *   [BLOG] "AI infra 学习记录(2): 从 LayerNorm 算子熟悉常见的算子优化方法"
 *   [LLMC] "02 · llmc/ 的 CUDA kernel 层" (llm.c CUDA kernel walk-through)
 *   [FP]   "GPU Performance from First Principles" (CS349D prerequisite
 *          lecture P1)
 *
 * Common conventions for every entry point
 * ----------------------------------------
 * Layout.  Every tensor of shape [rows, cols] is row-major and contiguous
 *   (row r starts at element r*cols).  gamma, beta and bias are [cols].
 *   mean, rstd are [rows] float32; dgamma, dbeta are [cols] float32.
 *   Storage type T of the [rows, cols] tensors and of gamma/beta/bias is
 *   given by `dt`; all arithmetic is float32 (the pages compute norms in
 *   FP32 and store FP16/BF16, [L10] §4.2).  Results are rounded to T with
 *   round-to-nearest-even.
 * Pointers.  All data pointers are DEVICE pointers (hipMalloc'd or equivalent)
 *   owned by the caller.  The library never allocates, frees or retains a
 *   pointer after the call returns.  No alignment is required: 16-byte
 *   aligned bases with cols*sizeof(T) a multiple of 16 take the vector path,
 *   anything else a per-element path with identical results.
 * Aliasing.  An output [rows, cols] tensor may be exactly one of the call's
 *   [rows, cols] inputs (in place: y == x, residual_out == residual,
 *   dx == dy, ...); every row is read completely before any of it is
 *   written.  Any other overlap of an output with an input or with another
 *   output is rejected with LN_ERR_UNSUPPORTED.
 * Streams.  All work is enqueued on `stream` (NULL = the null stream).  No
 *   call synchronises, allocates, memsets or copies, so every call may be
 *   captured into a HIP graph.  Outputs are valid once the stream has
 *   reached the enqueued work.
 * Errors.  Every call returns an ln_status_t.  All arguments are checked on
 *   the host before anything is enqueued, so a call that returns an error
 *   other than LN_ERR_HIP has written nothing.  rows == 0 is a no-op that
 *   returns LN_OK.  Launch failures are reported as LN_ERR_HIP.  No call
 *   prints, exits or throws.
 * Determinism.  Every output is bitwise reproducible from run to run on the
 *   same device for the same inputs and shape; dgamma/dbeta use a fixed
 *   partition of rows (a pure function of rows and cols) and a fixed-order
 *   fold, never floating-point atomics ([L11] §2.4 and [L10] §5.1 note that
 *   atomic accumulation order varies from run to run).
 * Tracing.  With MBROW_ROCTX=1 in the environment (read once per process),
 *   every entry point below that runs the library's row kernels (all but the
 *   streaming references hbm_copy and hbm_stream) opens a roctx range named
 *   after itself and closes it on return (rocprofv3 --marker-trace shows
 *   them); otherwise the library makes no roctx call.
 */
#ifndef MBROW_LN_H
#define MBROW_LN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LN_F32 = 0, LN_F16 = 1, LN_BF16 = 2 } ln_dtype_t;

typedef enum {
    LN_OK = 0,
    LN_ERR_NULL = 1,        /* a required pointer is NULL                      */
    LN_ERR_SHAPE = 2,       /* rows < 0 or cols <= 0                           */
    LN_ERR_DTYPE = 3,       /* unknown ln_dtype_t                              */
    LN_ERR_PARAM = 4,       /* eps < 0 or NaN; p outside [0, 1) or NaN         */
    LN_ERR_WORKSPACE = 5,   /* workspace smaller than ln_bwd_workspace_bytes   */
    LN_ERR_UNSUPPORTED = 6, /* cols above the call's LN_MAX_COLS*, or an
                               aliasing form the call does not allow          */
    LN_ERR_HIP = 7,         /* a HIP launch or query failed                    */
    LN_ERR_SCRATCH = 8      /* ln_bwd_noalloc: the shape needs more than the
                               library's static scratch of
                               LN_NOALLOC_SCRATCH_BYTES                       */
} ln_status_t;

/* Size of the static device scratch that ln_bwd_noalloc uses (per GPU, held
 * until the process ends). */
#define LN_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Widest row of ln_fwd and bias_dropout_residual_ln_fwd, for every storage
 * type.  Rows of up to 16384 columns are held in registers; wider rows are
 * staged in the LDS of one workgroup (read from global memory once while
 * they fit it: 39936 fp32 or 65536 16-bit columns; the rest of a wider fp32
 * row is read again in each later pass). */
#define LN_MAX_COLS 65536
/* Widest row of ln_bwd_dx, ln_bwd_dgamma_dbeta and ln_bwd_noalloc: past
 * 16384 columns both dy and x are staged in LDS, which holds 19968 fp32 or
 * (capped here) 32768 16-bit columns of each. */
#define LN_MAX_COLS_BWD_F32 19968
#define LN_MAX_COLS_BWD_16 32768
/* Widest row of add_rmsnorm_fwd and add_rmsnorm_bwd (registers only). */
#define LN_MAX_COLS_RMSNORM 16384
/* Widest row of bias_dropout_residual_ln_bwd, for every storage type (its
 * three column accumulators per value need the registers of twice as many
 * lanes). */
#define LN_MAX_COLS_DROPOUT_BWD 8192
/* Widest padded row (ld) of cross_entropy_fwd_bwd held in registers (and so
 * read once): 65536 fp32 or 163840 fp16/bf16 classes (the row is held in
 * the registers of one 1024-lane workgroup; GPT-2's 50257, Llama-3's 128256
 * and Qwen-2's 151936 classes fit in bf16). */
#define LN_MAX_COLS_XENT_F32 65536
#define LN_MAX_COLS_XENT_16 163840
/* Widest padded row (ld) of cross_entropy_fwd_bwd held on chip by one
 * workgroup, part in registers and part in LDS, and so still read once:
 * 131072 fp32 or 262144 fp16/bf16 classes (Llama-3's 128256 in fp32, a
 * 256000-class vocabulary in bf16).  Only rows on the 16-byte vector path (logits and dlogits
 * 16-byte aligned, ld * sizeof(T) a multiple of 16); other rows past
 * LN_MAX_COLS_XENT_* take the two-pass path. */
#define LN_MAX_COLS_XENT_LDS_F32 131072
#define LN_MAX_COLS_XENT_LDS_16 262144
/* Widest row of attn_softmax_fwd / attn_softmax_bwd held in registers (and
 * so read once): 32768 fp32 or 65536 fp16/bf16 scores (one 1024-lane
 * workgroup per row beyond 16384). */
#define LN_MAX_COLS_SOFTMAX_F32 32768
#define LN_MAX_COLS_SOFTMAX_16 65536
/* Widest row of attn_softmax_fwd still held on chip (read once) when its
 * rows are on the 16-byte vector path (x, mask, y and y_dropped 16-byte
 * aligned, cols * sizeof(T) a multiple of 16), with or without a mask row and
 * the dropped copy: 65536 fp32 / 131072 fp16/bf16 scores (1024 lanes x 16
 * slots of scores in registers; a mask row in registers and LDS).  Other
 * rows past LN_MAX_COLS_SOFTMAX_F32 / _16 take the two-pass path. */
#define LN_MAX_COLS_SOFTMAX_PLAIN_FWD_F32 65536
#define LN_MAX_COLS_SOFTMAX_PLAIN_FWD_16 131072
/* Widest row of attn_softmax_bwd held on chip (dy in registers, y in
 * registers and LDS, each read once, with or without dropout) when its rows
 * are on the 16-byte vector path: 65536 fp32 / 131072 fp16/bf16 scores.
 * Other rows past LN_MAX_COLS_SOFTMAX_F32 / LN_MAX_COLS_SOFTMAX_BWD_16 take
 * the two-pass path. */
#define LN_MAX_COLS_SOFTMAX_PLAIN_BWD_F32 65536
#define LN_MAX_COLS_SOFTMAX_PLAIN_BWD_16 131072
/* The same for attn_softmax_bwd with fp16/bf16 storage (it holds two
 * tensors, dy and y, per row). */
#define LN_MAX_COLS_SOFTMAX_BWD_16 49152
/* Widest row of attn_softmax_fwd / attn_softmax_bwd / cross_entropy_fwd_bwd:
 * rows wider than their on-chip paths (LN_MAX_COLS_SOFTMAX_* for the
 * softmax, LN_MAX_COLS_XENT_LDS_* on the vector path and LN_MAX_COLS_XENT_*
 * otherwise for the cross-entropy) take a two-pass path that reads the rest
 * of the row twice. */
#define LN_MAX_COLS_STREAM (1 << 24)

/*
 * LayerNorm forward.  For each row r with m = cols:
 *   mu = (1/m) sum_j x_j,  var = (1/m) sum_j (x_j - mu)^2,
 *   rstd = 1/sqrt(var + eps),  y_j = gamma_j * (x_j - mu) * rstd + beta_j.
 * [L11] §2.1 (xhat, sigma = sqrt(var + eps), save mu and r = 1/sigma);
 * [L10] §4.2 (population variance, one reduction); [BLOG] §2.1 gives the
 * same argument list (input, output, gamma, beta, rows, cols, eps).
 *   x     [rows, cols] T, input.
 *   gamma [cols] T, beta [cols] T.
 *   y     [rows, cols] T, output; may equal x.
 *   mean, rstd  [rows] float32 outputs, each may be NULL (inference keeps
 *         no intermediates, [L10] §6.3).
 *   eps   >= 0, added to the variance inside the square root.
 */
ln_status_t ln_fwd(const void* x, const void* gamma, const void* beta,
                   void* y, float* mean, float* rstd,
                   int64_t rows, int64_t cols, float eps, ln_dtype_t dt,
                   hipStream_t stream);

/*
 * Fused bias + dropout + residual + LayerNorm forward ([L10] §2.3: add the
 * bias, apply dropout, add the residual, in one kernel; [LLMC] §3.2: the
 * residual sum is written out and normalised in the same kernel).
 *   t = x + bias;  keep = mask(seed, r, j, p);
 *   z = residual + (keep ? t / (1 - p) : 0)     (inverted dropout);
 *   residual_out = round_T(z);  then LayerNorm of the stored residual_out,
 *   exactly as ln_fwd(residual_out) would compute it.
 * The mask is a pure function of (seed, row, column, p), so a backward pass
 * regenerates it from the seed instead of storing it ([L11] §3.3):
 *   key = (seed & 0xffffffff, seed >> 32), counter = (col >> 3,
 *   row & 0xffffffff, row >> 32, 0), w = Philox4x32-10(counter, key)
 *   (Salmon et al., SC'11); u = 16-bit half (col & 1) of word (col & 7) >> 1;
 *   keep iff u >= floor(p * 65536 + 0.5) evaluated in double from float p.
 *   x, residual  [rows, cols] T inputs;  bias, gamma, beta [cols] T.
 *   residual_out [rows, cols] T output (z).   y [rows, cols] T output.
 *   mean, rstd   [rows] float32 outputs of the LayerNorm of z, nullable.
 *   mask_out     [rows, cols] uint8 output (1 = kept), nullable; debugging
 *                and tests only, the mask never needs to be stored.
 *   p in [0, 1): dropout probability; seed: 64-bit mask seed.
 */
ln_status_t bias_dropout_residual_ln_fwd(
    const void* x, const void* bias, const void* residual,
    const void* gamma, const void* beta, void* residual_out, void* y,
    float* mean, float* rstd, uint8_t* mask_out,
    int64_t rows, int64_t cols, float eps, float p, uint64_t seed,
    ln_dtype_t dt, hipStream_t stream);

/*
 * Bytes of float32 workspace the backward needs for the per-partition
 * column partials of dgamma and dbeta: P * 2 * cols * 4, where the number of
 * row partitions P depends only on (rows, cols).  Returns 0 for rows <= 0 or
 * cols <= 0.  ([L11] §2.4: split the rows into P ranges, one partial sum per
 * range, then a second small kernel adds the P partials.)
 */
size_t ln_bwd_workspace_bytes(int64_t rows, int64_t cols);

/*
 * LayerNorm backward, input gradient, with both row sums in one reduction
 * ([L11] §2.1 "HW4" form, §2.2 one synchronisation):
 *   g_j = gamma_j * dy_j,  xhat_j = (x_j - mean) * rstd,
 *   A = sum_j g_j,  B = sum_j g_j * xhat_j,
 *   dx_j = rstd * (g_j - (A + xhat_j * B) / cols).
 *   dy, x [rows, cols] T inputs;  gamma [cols] T;
 *   mean, rstd [rows] float32 as saved by the forward;
 *   dx [rows, cols] T output; may equal dy.
 *   workspace  float32 device buffer or NULL.  When non-NULL the same pass
 *              also writes the stage-1 column partials of dgamma/dbeta
 *              (dgamma = sum_rows dy * xhat, dbeta = sum_rows dy, [L11]
 *              §2.1/§2.4) into it; finish them with
 *              ln_bwd_dgamma_dbeta(..., partials_ready = 1, ...).
 *   workspace_bytes  its size; must be >= ln_bwd_workspace_bytes(rows, cols)
 *              when workspace is non-NULL.
 */
ln_status_t ln_bwd_dx(const void* dy, const void* x, const void* gamma,
                      const float* mean, const float* rstd, void* dx,
                      float* workspace, size_t workspace_bytes,
                      int64_t rows, int64_t cols, ln_dtype_t dt,
                      hipStream_t stream);

/*
 * LayerNorm backward, parameter gradients (column sums over rows, [L11]
 * §2.1 and §2.4): dgamma_j = sum_r dy_rj * xhat_rj, dbeta_j = sum_r dy_rj,
 * as float32, by a deterministic two-stage reduction: P per-partition
 * partials, then a fixed-order fold.
 *   partials_ready = 1: the workspace already holds the partials written by
 *     ln_bwd_dx for the same (rows, cols); only the fold runs, and dy, x,
 *     mean, rstd may be NULL.
 *   partials_ready = 0: stage 1 runs here first (reads dy, x, mean, rstd);
 *     the result is bitwise identical to the ln_bwd_dx path.
 *   dgamma, dbeta [cols] float32 outputs.
 *   workspace / workspace_bytes as for ln_bwd_dx (required here).
 */
ln_status_t ln_bwd_dgamma_dbeta(const void* dy, const void* x,
                                const float* mean, const float* rstd,
                                float* dgamma, float* dbeta,
                                float* workspace, size_t workspace_bytes,
                                int partials_ready, int64_t rows,
                                int64_t cols, ln_dtype_t dt,
                                hipStream_t stream);

/*
 * The whole LayerNorm backward -- dx, dgamma and dbeta -- for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments and results as
 * ln_bwd_dx with a workspace followed by ln_bwd_dgamma_dbeta with
 * partials_ready = 1 (the same kernels: results are bitwise identical), but
 * the column partials live in a static device array of the library,
 * LN_NOALLOC_SCRATCH_BYTES per GPU, instead of a caller workspace.  The call
 * allocates nothing and calls no allocating routine.
 *   Shapes whose partials need more than LN_NOALLOC_SCRATCH_BYTES
 *   (ln_bwd_workspace_bytes(rows, cols) > LN_NOALLOC_SCRATCH_BYTES, e.g. more
 *   than 8192 columns at 256 rows or more) return LN_ERR_SCRATCH and enqueue
 *   nothing.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on one
 *   GPU (concurrent streams, or host threads on the same device) race and
 *   must be serialised by the caller.  Nothing in the array needs clearing:
 *   each call writes every partial it later reads.
 */
ln_status_t ln_bwd_noalloc(const void* dy, const void* x, const void* gamma,
                           const float* mean, const float* rstd, void* dx,
                           float* dgamma, float* dbeta, int64_t rows, int64_t cols,
                           ln_dtype_t dt, hipStream_t stream);

/*
 * Bytes of float32 workspace bias_dropout_residual_ln_bwd needs: P * 3 * cols
 * * 4 (dgamma, dbeta and dbias partials per partition), with the same P as
 * ln_bwd_workspace_bytes.  Returns 0 for rows <= 0 or cols <= 0.
 */
size_t bias_dropout_residual_ln_bwd_workspace_bytes(int64_t rows, int64_t cols);

/*
 * Backward of bias_dropout_residual_ln_fwd in one pass over the rows: the
 * LayerNorm backward as in ln_bwd_dx / ln_bwd_dgamma_dbeta, then the
 * prologue's backward by the chain rule through
 * z = residual + keep * (x + bias) / (1 - p), with the forward's mask
 * regenerated from (seed, row, column, p) instead of stored ([L11] §3.3;
 * [L10] §2.3 for the order bias add, dropout, residual add):
 *   dz        = dx of the LayerNorm (from dy) + dz_extra;
 *   dresidual = dz;
 *   dx_j      = keep_j ? dz_j / (1 - p) : 0;
 *   dbias_j   = sum over rows of dx_j (before rounding to T), dgamma_j =
 *               sum dy * xhat, dbeta_j = sum dy, by the same deterministic
 *               two-stage reduction ([L11] §2.4).
 * dz is formed in float32; dresidual and dx are rounded from it.
 *   dy        [rows, cols] T: gradient of y.
 *   dz_extra  [rows, cols] T or NULL: gradient reaching z from its other
 *             uses (the residual stream); NULL adds nothing.
 *   z         [rows, cols] T: residual_out of the forward.
 *   gamma [cols] T;  mean, rstd [rows] float32 as saved by the forward.
 *   p, seed   the forward's dropout probability and seed.
 *   dresidual, dx  [rows, cols] T outputs; each may equal exactly one of dy,
 *             dz_extra, z (in place), but not each other.
 *   dgamma, dbeta, dbias  [cols] float32 outputs.
 *   workspace float32 device buffer of at least
 *             bias_dropout_residual_ln_bwd_workspace_bytes(rows, cols).
 * Errors as for the other calls; p outside [0, 1) is LN_ERR_PARAM; rows wider
 * than LN_MAX_COLS_DROPOUT_BWD are LN_ERR_UNSUPPORTED.
 */
ln_status_t bias_dropout_residual_ln_bwd(const void* dy, const void* dz_extra, const void* z,
                                         const void* gamma, const float* mean,
                                         const float* rstd, void* dresidual, void* dx,
                                         float* dgamma, float* dbeta, float* dbias,
                                         float* workspace, size_t workspace_bytes,
                                         int64_t rows, int64_t cols, float p, uint64_t seed,
                                         ln_dtype_t dt, hipStream_t stream);

/*
 * The two stages of bias_dropout_residual_ln_bwd as separate calls (as
 * ln_bwd_dx and ln_bwd_dgamma_dbeta split the LayerNorm backward), for callers
 * that schedule the small second stage themselves:
 *   bias_dropout_residual_ln_bwd_dx writes dresidual, dx and the column
 *     partials of dgamma, dbeta and dbias into the workspace (arguments and
 *     errors as for bias_dropout_residual_ln_bwd, without the [cols] outputs);
 *   bias_dropout_residual_ln_bwd_fold adds those partials for the same
 *     (rows, cols) in the fixed order into dgamma, dbeta, dbias ([cols]
 *     float32).  rows < 0 or cols <= 0 is LN_ERR_SHAPE, cols above
 *     LN_MAX_COLS_DROPOUT_BWD LN_ERR_UNSUPPORTED.
 * The two calls in turn give bitwise the results of the combined call.
 */
ln_status_t bias_dropout_residual_ln_bwd_dx(const void* dy, const void* dz_extra, const void* z,
                                            const void* gamma, const float* mean,
                                            const float* rstd, void* dresidual, void* dx,
                                            float* workspace, size_t workspace_bytes,
                                            int64_t rows, int64_t cols, float p, uint64_t seed,
                                            ln_dtype_t dt, hipStream_t stream);
ln_status_t bias_dropout_residual_ln_bwd_fold(const float* workspace, size_t workspace_bytes,
                                              float* dgamma, float* dbeta, float* dbias,
                                              int64_t rows, int64_t cols, hipStream_t stream);

/*
 * Attention softmax forward over rows of `cols` scores ([L10] §4.1: per row,
 * scale, add the mask, subtract the row maximum, exp, divide by the row sum;
 * one row per group of lanes, held in registers):
 *   t_j = scale * x_j + mask[r / rows_per_mask][j]   (mask NULL: no term);
 *   causal = 1: t_j = -inf for keys j > q, q = r mod cols (rows are square
 *               [L, L] score blocks one after another; keys past the query
 *               are not read);
 *   y_j = exp(t_j - max t) / sum_k exp(t_k - max t); a row whose every key
 *   is masked gives y = 0.
 *   y_dropped_j = keep_j ? y_j / (1 - p) : 0 with the same mask function of
 *   (seed, row, column, p) as bias_dropout_residual_ln_fwd; NULL skips it.
 *   x [rows, cols] T input;  mask [ceil(rows / rows_per_mask), cols] T or
 *   NULL;  y [rows, cols] T output (may equal x);  y_dropped [rows, cols] T
 *   output or NULL (may equal x, not y).
 * scale must be finite; causal 0 or 1; p in [0, 1); rows_per_mask >= 1 when
 * mask is given.  Arithmetic in float32 (exp by the device's exp2).  Rows of
 * up to LN_MAX_COLS_SOFTMAX_F32 (fp32) or LN_MAX_COLS_SOFTMAX_16 (fp16/bf16)
 * columns are held in registers (read once), and rows of up to
 * LN_MAX_COLS_SOFTMAX_PLAIN_FWD_F32 / _16 columns on the vector path are held
 * on chip (the scores in registers, a mask row in registers and LDS); wider
 * rows, up to LN_MAX_COLS_STREAM, are read twice: an online maximum/sum pass
 * ([LLMC] §6.1), then the output pass.
 */
ln_status_t attn_softmax_fwd(const void* x, const void* mask, int64_t rows_per_mask, void* y,
                             void* y_dropped, int64_t rows, int64_t cols, float scale,
                             int causal, float p, uint64_t seed, ln_dtype_t dt,
                             hipStream_t stream);

/*
 * Attention softmax backward fused with the attention-dropout backward
 * ([L11] §3: the dropout backward in registers first, then one dot product
 * per row):  g_j = keep_j ? dy_j / (1 - p) : 0 (the forward's mask
 * regenerated; p = 0 keeps all), s = sum_j g_j * y_j,
 * dx_j = scale * y_j * (g_j - s).
 *   dy [rows, cols] T: gradient of y_dropped (of y when p = 0).
 *   y  [rows, cols] T: the forward's y.   dx [rows, cols] T output (may equal
 *   dy or y).  causal = 1 skips reading the keys past the query (y = 0
 *   there, so dx = 0).  Rows wider than LN_MAX_COLS_SOFTMAX_F32 (fp32) or
 *   LN_MAX_COLS_SOFTMAX_BWD_16 (fp16/bf16), up to LN_MAX_COLS_STREAM, read dy
 *   and y twice: the dot product, then dx; rows on the vector path are
 *   held on chip and read once up to LN_MAX_COLS_SOFTMAX_PLAIN_BWD_F32 / _16
 *   (with dropout, the keep bits are regenerated from the seed on chip).
 */
ln_status_t attn_softmax_bwd(const void* dy, const void* y, void* dx, int64_t rows,
                             int64_t cols, float scale, int causal, float p, uint64_t seed,
                             ln_dtype_t dt, hipStream_t stream);

/*
 * Fused residual add + RMSNorm forward ([FP] §6.1: the residual add and the
 * next RMSNorm as one kernel that reads x and the residual and writes the new
 * residual stream and the normalised h).  For each row r with m = cols:
 *   z_j  = x_j + residual_j, rounded to T (residual NULL: z = x, nothing
 *          written to residual_out);
 *   rstd = 1 / sqrt(sum_j z_j^2 / m + eps), on the rounded z, in float32
 *          ([FP] §7.5: the sum of squares is float32 because squares of
 *          activation outliers of a few hundred overflow fp16);
 *   y_j  = z_j * rstd * gamma_j.
 *   x, residual    [rows, cols] T inputs (residual may be NULL).
 *   gamma          [cols] T.
 *   residual_out   [rows, cols] T output z; required with a residual, must be
 *                  NULL without one (LN_ERR_PARAM); may equal x or residual.
 *   y              [rows, cols] T output; may equal x or residual, not
 *                  residual_out.
 *   rstd           [rows] float32 output, or NULL (inference).
 * eps >= 0 and finite, else LN_ERR_PARAM.
 */
ln_status_t add_rmsnorm_fwd(const void* x, const void* residual, const void* gamma,
                            void* residual_out, void* y, float* rstd, int64_t rows, int64_t cols,
                            float eps, ln_dtype_t dt, hipStream_t stream);

/*
 * Bytes of float32 workspace add_rmsnorm_bwd needs: P * cols * 4 (dgamma
 * partials per partition), with the same P as ln_bwd_workspace_bytes.
 * Returns 0 for rows <= 0 or cols <= 0.
 */
size_t add_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t cols);

/*
 * Backward of add_rmsnorm_fwd.  With g = gamma * dy and xhat = z * rstd
 * (RMSNorm is the LayerNorm of [L11] §2.1 with the mean fixed at 0, so the
 * sum of g drops out):
 *   dz_j     = rstd * (g_j - xhat_j * sum_k g_k xhat_k / m) + dz_extra_j,
 *              one row sum per row, formed in float32 and rounded to T once;
 *              it is the gradient of both x and residual of the forward;
 *   dgamma_j = sum over rows of dy * xhat, float32, by the deterministic
 *              two-stage reduction of ln_bwd_dgamma_dbeta ([L11] §2.4).
 *   dy        [rows, cols] T: gradient of y.
 *   dz_extra  [rows, cols] T or NULL: gradient reaching z from its other
 *             uses (the residual stream); NULL adds nothing.
 *   z         [rows, cols] T: residual_out of the forward (x without a
 *             residual).
 *   gamma [cols] T;  rstd [rows] float32 as saved by the forward.
 *   dz        [rows, cols] T output; may equal exactly one of dy, dz_extra
 *             or z (in place).
 *   dgamma    [cols] float32 output.
 *   workspace float32 device buffer of at least
 *             add_rmsnorm_bwd_workspace_bytes(rows, cols).
 * Errors as for the other calls.
 */
ln_status_t add_rmsnorm_bwd(const void* dy, const void* dz_extra, const void* z,
                            const void* gamma, const float* rstd, void* dz, float* dgamma,
                            float* workspace, size_t workspace_bytes, int64_t rows, int64_t cols,
                            ln_dtype_t dt, hipStream_t stream);

/*
 * Cross-entropy with label smoothing, forward and backward in one pass over
 * each row of logits ([L10] §5.2: with q = softmax(x) and the smoothed target
 * p_j = (1 - a)[j == label] + a/V, the loss is
 * log Z + m - [(1 - a) x_label + (a/V) sum_j x_j] (m the row maximum,
 * Z = sum_j exp(x_j - m)) and its gradient is q - p; [LLMC] §6.1: the row's
 * maximum and exp-sum from one online softmax reduction, the probabilities
 * never stored, the gradient written over the logits in the same kernel):
 *   loss_r   = the label-smoothed cross-entropy of row r (float32);
 *   dlogits  = grad_scale * (q - p), rounded to T.
 *   logits   [rows, ld] T; columns [0, cols) are the V = cols classes,
 *            columns [cols, ld) are padding and are never read.
 *   labels   [rows] int64 class indices.  A negative label marks an ignored
 *            row: loss 0, gradient 0.  A label >= cols has no target: loss
 *            and the row's gradient are NaN.
 *   loss     [rows] float32 output.
 *   dlogits  [rows, ld] T output or NULL (loss only); may equal logits (in
 *            place).  Its padding columns are written with 0.
 *   label_smoothing a in [0, 1];  grad_scale finite (e.g. 1/rows for a mean
 *            loss).
 * ld >= cols, else LN_ERR_SHAPE.  Rows of up to LN_MAX_COLS_XENT_F32 (fp32) or
 * LN_MAX_COLS_XENT_16 (fp16/bf16) columns are held in registers and read
 * once; on the 16-byte vector path, rows of up to LN_MAX_COLS_XENT_LDS_F32 /
 * LN_MAX_COLS_XENT_LDS_16 are held in the registers and LDS of one workgroup
 * and still read once; wider rows, up to LN_MAX_COLS_STREAM (else
 * LN_ERR_UNSUPPORTED), are read twice: an online maximum/sum pass, then the
 * gradient pass.
 * Arithmetic in float32 (exp by the device's exp2).
 */
ln_status_t cross_entropy_fwd_bwd(const void* logits, const int64_t* labels, float* loss,
                                  void* dlogits, int64_t rows, int64_t cols, int64_t ld,
                                  float label_smoothing, float grad_scale, ln_dtype_t dt,
                                  hipStream_t stream);

/*
 * Measurement reference, not a step of any method: copies `bytes` bytes from
 * src to dst (device pointers) in 16-byte vectors with nontemporal loads and
 * stores (hbm_stream with one source and one destination), the
 * attainable-bandwidth figure that the row kernels' rates are compared
 * against.  bytes, src and dst must be multiples of 16 and the two
 * ranges must not overlap, else LN_ERR_PARAM; NULL with bytes > 0 is
 * LN_ERR_NULL; bytes == 0 is a no-op.  Enqueued on `stream`; no allocation.
 */
ln_status_t hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/*
 * Measurement reference, not a step of any method: reads nsrc (1..3) tensors
 * of `bytes` bytes each and writes ndst (0..2) tensors of the same size (the
 * xor and the sum of the sources' 16-byte vectors), one 16-byte vector per
 * tensor per thread with nontemporal accesses -- the attainable bandwidth of
 * a kernel that streams the same mix of reads and writes (a LayerNorm
 * forward reads 1 tensor and writes 1; the fused forward 2 and 2; the
 * backward 2 and 1; the prologue backward 3 and 2).  src and dst are HOST
 * arrays of nsrc and ndst device pointers.  nsrc or ndst out of range, bytes
 * or a pointer not a multiple of 16, or a destination overlapping a source or
 * another destination is LN_ERR_PARAM; a NULL array or pointer LN_ERR_NULL;
 * bytes == 0 a no-op.  Enqueued on `stream`; no allocation.
 */
ln_status_t hbm_stream(const void* const* src, int nsrc, void* const* dst, int ndst,
                       size_t bytes, hipStream_t stream);

/* Static English description of a status code (never NULL). */
const char* ln_status_string(ln_status_t status);

#ifdef __cplusplus
}
#endif

#endif
