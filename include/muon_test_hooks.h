/* muon_test_hooks.h -- host-only hooks of libmuon for the test suite.
 *
 * These entry points are not part of the product interface in muon.h: they expose the
 * tile orders, the tail split and the operand-addressing switch of the MFMA kernels so that
 * tests can check them on the host, and they may change with the kernels.  Same conventions
 * as muon.h (C ABI, status codes); none of them enqueues GPU work.
 */
#ifndef MUON_TEST_HOOKS_H
#define MUON_TEST_HOOKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Test hooks (host only): the tile orders used by the MFMA kernel.
 * muon_debug_tile_order: tile t of one matrix -> (ti[t], tj[t]); tri != 0 walks the lower
 * triangle of a tm x tm tile grid, else the full tm x tn grid.  Returns the tile count;
 * ti and tj must hold that many ints.
 * muon_debug_xcd_remap: workgroup w -> logical tile out[w] for a grid of `total`. */
int muon_debug_tile_order(int tri, int tm, int tn, int* ti, int* tj);
int muon_debug_xcd_remap(int total, int* out);
/* muon_debug_wide_tile_order: the same for the 256 x 384 configuration over a rows x cols
 * output: tri != 0 walks the 256 x 384 tiles that meet the lower triangle of a rows x rows
 * output (ti: 256-row band, tj: 384-column band).  Returns the tile count. */
int muon_debug_wide_tile_order(int tri, int rows, int cols, int* ti, int* tj);
/* muon_debug_split: the tail split of a launch of `tiles` tiles on `units` compute units
 * whose tail tiles have `ksteps` k-steps each.  plan[0..5] receives the mode (0 none,
 * 1 equal pieces, 2 one uneven cut), the pieces per tail tile (mode 1) or the cut's second
 * pieces per unit (mode 2), the workgroups running whole tiles, the tail tiles, the tail
 * workgroups and the partial-sum slots.  When items is not NULL, items[5 j .. 5 j + 4]
 * receives, for tail workgroup j < max_items, its tail tile, piece, piece count and k-step
 * range [k0, k1), or -1 in the first field for a workgroup without a piece.  Returns the
 * number of tail workgroups, or MUON_EINVAL for a NULL plan or negative sizes. */
int muon_debug_split(int tiles, int units, int ksteps, int* plan, int* items, int max_items);
/* muon_debug_flat_loads: on != 0 makes every later launch of the 256 x 256 MFMA kernel and of
 * its deep-pipeline and 128 x 128 builds (of muon_step and shampoo_step) address its operands
 * with 64-bit pointers, the path it otherwise takes only
 * when an operand of the launch is 2 GB or larger (below that it uses 32-bit buffer
 * offsets); 0 restores the default.  Process-wide.  For tests of that path. */
int muon_debug_flat_loads(int32_t on);
/* muon_debug_split_spins: polls of a tail-split last piece's bounded wait for every later MFMA
 * launch (spins >= 0); -1 restores the default (about a second); -2 never polls, so every
 * such wait times out at once: the timeout path runs on the GPU with no wait at all.
 * Process-wide.  MUON_EINVAL below -2. */
int muon_debug_split_spins(int32_t spins);
/* muon_debug_split_protocol: runs the tail split's counter protocol (arrive, publish, collect)
 * for one tile of `pieces` pieces (2..8) on the host, with the library's own protocol code
 * over host atomics.  mode 0: each piece on its own thread; 2: the pieces in order; 1: in
 * order, but piece 0 publishes only after the last piece's wait of `spin_limit` polls ran
 * out, and then a later launch's pieces arrive on the same counters.  spin_limit -1 never
 * polls (as the kernels under muon_debug_split_spins(-2)).  out[0..7]: pieces that
 * took the last-piece role, collect succeeded (1/0), cnt[0] and cnt[1] after, the status
 * word, slots the last piece saw written (itself included), and for mode 1 cnt[1] after the
 * late publish and the later launch's pieces that took the last-piece role (else -1). */
int muon_debug_split_protocol(int32_t pieces, int32_t mode, int32_t spin_limit, int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* MUON_TEST_HOOKS_H */
