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
/* muon_debug_flat_loads: on != 0 makes every later 256 x 256 MFMA launch (of muon_step and
 * shampoo_step) address its operands with 64-bit pointers, the path it otherwise takes only
 * when an operand of the launch is 2 GB or larger (below that it uses 32-bit buffer
 * offsets); 0 restores the default.  Process-wide.  For tests of that path. */
int muon_debug_flat_loads(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* MUON_TEST_HOOKS_H */
