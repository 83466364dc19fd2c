/*
 * fa_debug.h -- entry point of the DEBUG build of libfa_mi355x
 * (libfa_mi355x_debug.so, compiled with FA_DEBUG_BUILD=1); the production
 * library does not export it.
 *
 * The debug build computes the same results as the production library (its
 * kernels are the same code) and adds two checks:
 *   - every tiled kernel fills its LDS with a quiet NaN before first use, so
 *     a read of LDS that was never written would show in the outputs;
 *   - the forward, dQ and dK/dV kernels count the tiles they load into a
 *     caller's array, so a test can compare which tiles are touched with
 *     which the visibility rules need (only kept blocks of a block-sparse
 *     mask, and no key tile that no row of a query tile sees -- the
 *     block-sparse paragraph of the agihunt.info summary of the paper; the
 *     causal-mask section of the marketmaker.cc article).
 */
#ifndef FA_MI355X_DEBUG_H
#define FA_MI355X_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sets (NULL: clears) the device array that later fa_fwd / fa_bwd /
 * fa_bwd_dq / fa_bwd_dkdv calls of this process add tile visits to; the
 * caller zeroes it and keeps it alive.  Layout, int32, with nb = ceil(N / 128)
 * and BH = B * H query heads:
 *   [0][BH][nb][nb]   forward:  [head][128-row query tile][128-key block]
 *                     += keys of each key tile the workgroup loads;
 *   [1][BH][nb][nb]   dQ kernel, the same;
 *   [2][BH][nb][nb]   dK/dV kernel: [query head][128-key tile][128-query
 *                     block] += queries of each query step loaded for it.
 * Not thread-safe (process-wide setting of a debug library).  Returns FA_OK. */
int fa_debug_set_tile_visits(int32_t* visits);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_DEBUG_H */
