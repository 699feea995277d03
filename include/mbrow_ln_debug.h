/*
 * mbrow_ln_debug.h -- test-only controls of the fused LayerNorm library.
 *
 * The library picks, per call, how many lanes own a row (16, 32 or 64 lanes
 * of one wave, or 2-16 waves of one workgroup) and how many 16-byte slots each
 * lane holds, from the storage type and the row width.  Tests force other
 * choices on the same shape to check that every path computes the same
 * results; a production caller never needs this.
 */
#ifndef MBROW_LN_DEBUG_H
#define MBROW_LN_DEBUG_H

#include "mbrow_ln.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Force the row layout of every later call in this process:
 *   lanes_per_row  16, 32, 64, 128, 256, 512 or 1024; 0 restores the
 *                  library's own choice (and ignores slots_per_lane).
 *   slots_per_lane 16-byte slots per lane.  Built layouts: fp32 16x{1,2,4,8},
 *                  32x1-8, 64x1-8, {128,256,512,1024}x4; fp16/bf16
 *                  16x{1,2,4}, 32x1-5, 64x1-5, {128,256,512}x4.  The attention
 *                  softmax also has 1024x5-8 (fp32) and 512x{6,8}, 1024x3-8
 *                  (fp16/bf16; its backward 1024x3-6), the cross-entropy its
 *                  own set (1024 x up to 16 fp32, 20 fp16/bf16).  The prologue
 *                  backward (bias_dropout_residual_ln_bwd) has its own set:
 *                  fp32 16x{1,2,4}, 32x1-4, 64x1-6, {128,256,512}x4;
 *                  fp16/bf16 16x{1,2}, 32x1-3, 64x1-3, {128,256,512}x2.
 *   scalar         non-zero forces per-element loads and stores.
 * A forced layout applies only to calls that have it built for their dtype
 * and whose row fits it (lanes_per_row * slots_per_lane slots); other calls
 * use the library's own choice.  Returns LN_ERR_UNSUPPORTED (and changes nothing)
 * for a layout no dtype was built with.  Not thread-safe with respect to concurrent
 * calls that expect a particular layout.
 */
ln_status_t ln_debug_force_path(int lanes_per_row, int slots_per_lane, int scalar);

/*
 * Force the grid of the persistent forward kernels: workgroups_per_cu > 0
 * launches that many workgroups per compute unit, -1 one workgroup per block
 * of rows (no persistence), 0 restores the occupancy-derived default.
 * Results do not depend on it.
 */
ln_status_t ln_debug_force_grid(int workgroups_per_cu);

/*
 * on != 0: every later attn_softmax_fwd / attn_softmax_bwd /
 * cross_entropy_fwd_bwd call takes the two-pass path (the one for rows wider
 * than the register layouts) whatever its width; 0 restores the width-based
 * choice.  Results are within the same tolerances either way.
 */
ln_status_t ln_debug_force_two_pass(int on);

/*
 * on != 0: every later ln_fwd, bias_dropout_residual_ln_fwd, ln_bwd_dx,
 * ln_bwd_dgamma_dbeta and ln_bwd_noalloc call takes the LDS-staged path (the
 * one for rows wider than 16384 columns) whatever its width; 0 restores the
 * width-based choice.  Results are within the same tolerances either way.
 */
ln_status_t ln_debug_force_staged(int on);

#ifdef __cplusplus
}
#endif

#endif
