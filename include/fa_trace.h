/*
 * fa_trace.h -- debug entry point of the trace build of the library
 * (libfa_trace.so: the same sources compiled with FA_TRACE_VISITS).
 *
 * It checks, on the device, the tile skipping of the varlen tile scheduler:
 * the pages fix which (query row, key) pairs each sparse mode allows
 * (aclnnFlashAttentionUnpaddingScoreGrad, sparseMode parameter list), and a
 * pass must compute exactly the tiles that hold at least one allowed pair.
 * In the trace build every kernel counts each tile it computes into a device
 * counter array of uint32; the product library (libfa.so) has no counters and
 * does not export this call.
 */
#ifndef FA_TRACE_H_
#define FA_TRACE_H_

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Sets (counters != NULL) or clears the visit counters of one pass for the
 * calls that follow:
 *   pass 0, fa_fwd:  one count per (32-row block, 64-key tile) a wave computes;
 *   pass 1, fa_bwd dK/dV pass: one count per (64-row tile, 128-key tile) step;
 *   pass 2, fa_bwd dQ pass: one count per (32-row block, 64-key tile).
 * Counter of (sequence b, query head h, row block r, key tile t):
 *   ((b * Nq + h) * RB + r) * KT + t, with RB / KT the block and tile counts of
 * the longest query / key sequence of the call.  The caller zeroes the array
 * (device memory of `words` uint32) and owns it; a call whose grid needs more
 * than `words` counters returns FA_ERR_PARAM_INVALID (in the trace build this
 * check runs after the work plan has been staged).  pass outside [0, 2] ->
 * FA_ERR_PARAM_INVALID.
 */
fa_status fa_debug_trace(int32_t pass, uint32_t* counters, int64_t words);

#ifdef __cplusplus
}
#endif

#endif /* FA_TRACE_H_ */
