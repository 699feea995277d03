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
 *   slots_per_lane 16-byte slots per lane: 1 for 16/32 lanes, 1-8 for 64,
 *                  4 for 128-512, 4 or 8 for 1024.
 *   scalar         non-zero forces per-element loads and stores.
 * A forced layout applies only to calls whose row fits it
 * (lanes_per_row * slots_per_lane slots); other calls use the library's own
 * choice.  Returns LN_ERR_UNSUPPORTED (and changes nothing) for a layout the
 * library was not built with.  Not thread-safe with respect to concurrent
 * calls that expect a particular layout.
 */
ln_status_t ln_debug_force_path(int lanes_per_row, int slots_per_lane, int scalar);

#ifdef __cplusplus
}
#endif

#endif
