// Counter protocol of a tile whose contraction the tail split cut into pieces (tile_order.h),
// written once for the kernels (device atomics) and for a host emulation (host atomics):
// `Ops` supplies fetch_add, load, store and pause on int32_t words.
//
// Per tail tile, two counters that are zero when a step's first launch has run:
//   1. arrive: a piece that has finished its part of the k loop counts itself in cnt[0]; the
//      one that sees pieces - 1 before its own count is the last piece;
//   2. publish: every other piece, once its fp32 partial sums are stored and complete,
//      counts them in cnt[1];
//   3. collect: the last piece waits until cnt[1] reaches pieces - 1, then clears both
//      counters for the next launch of the step and adds the partial sums.
// The wait in 3 is for pieces that have already passed step 1: they are running and need
// nothing from anyone to finish step 2, so it ends; it is bounded all the same.  If the
// bound is ever reached the last piece sets the workspace's sticky status word, leaves both
// counters as they are (a piece still to publish then counts into a pair nobody clears, and
// no later launch of the step can take a stale count for a complete one without the status
// word being set) and reports the timeout, and its caller stores NaN for the tile.
#pragma once

#include <cstdint>

#if defined(__HIP__)
#define MUON_SPLIT_HD __attribute__((host)) __attribute__((device)) inline
#else
#define MUON_SPLIT_HD inline
#endif

namespace muon {

constexpr int32_t kStatusSplitTimeout = 1;  // status word: a tail-split wait timed out
constexpr int kSplitSpins = 1 << 22;        // polls of the last piece's wait (about a second)

// Step 1 in two halves: the count the arriving piece saw, and whether that makes it the last.
template <typename Ops>
MUON_SPLIT_HD int32_t split_arrive_count(Ops& o, int32_t* cnt) {
  return o.fetch_add(&cnt[0], 1);
}
MUON_SPLIT_HD bool split_is_last(int32_t count, int pieces) { return count == pieces - 1; }

template <typename Ops>
MUON_SPLIT_HD bool split_arrive(Ops& o, int32_t* cnt, int pieces) {
  return split_is_last(split_arrive_count(o, cnt), pieces);
}

template <typename Ops>
MUON_SPLIT_HD void split_publish(Ops& o, int32_t* cnt) {
  o.fetch_add(&cnt[1], 1);
}

// Returns true when the other pieces' sums are complete (counters cleared), false on a
// timeout after `spin_limit` polls (status word set, counters kept).  A negative spin_limit
// never polls: every wait times out at once (tests force the timeout path with it).
template <typename Ops>
MUON_SPLIT_HD bool split_collect(Ops& o, int32_t* cnt, int pieces, int spin_limit, int32_t* status) {
  for (int spins = 0; spin_limit >= 0; ++spins) {
    if (o.load(&cnt[1]) >= pieces - 1) {
      o.store(&cnt[0], 0);
      o.store(&cnt[1], 0);
      return true;
    }
    if (spins >= spin_limit) break;
    o.pause();
  }
  o.store(status, kStatusSplitTimeout);
  return false;
}

}  // namespace muon
