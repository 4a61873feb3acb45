// Owner assignment for the owner-side step (DMuon summary §2.3): every matrix gets one owner
// rank, and the assignment minimises the predicted makespan, the largest total cost of one
// owner.  The costs are measured step times per matrix.  The summary poses the problem as a
// mixed-integer program, with a greedy heuristic for search spaces that are too large.  Here:
//   1. greedy longest-first: matrices in decreasing cost (ties in list order), each to the
//      owner with the smallest load so far (lowest index on ties);
//   2. for up to kExactMax matrices, an exact depth-first search over assignments that starts
//      from the greedy makespan and stops at a node budget.  When it completes, its result is
//      the optimum of the mixed-integer program.
// Host code only: no HIP call.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/muon.h"

namespace {

constexpr int kExactMax = 64;  // largest count the exact search is tried on

struct Search {
  const std::vector<double>* cost;  // in decreasing order
  int ranks = 0;
  int64_t node_limit = 0;
  int64_t nodes = 0;
  bool aborted = false;
  double best = 0.0;     // best makespan found so far (the greedy's to start with)
  double lower = 0.0;    // max(largest cost, total / ranks): no assignment does better
  std::vector<double> load;
  std::vector<int> cur, best_owner;
  std::vector<double> rem;  // rem[k] = sum of cost[k..]

  // Assign matrices k.. (in decreasing cost) given the loads so far; max_load is the
  // largest current load.
  void dfs(int k, double max_load, double sum_load) {
    if (aborted || best <= lower) return;
    if (++nodes > node_limit) {
      aborted = true;
      return;
    }
    const int n = int(cost->size());
    if (k == n) {
      if (max_load < best) {
        best = max_load;
        best_owner = cur;
      }
      return;
    }
    // No completion beats max(current max load, average load at the end).
    if (std::max(max_load, (sum_load + rem[k]) / ranks) >= best) return;
    const double c = (*cost)[k];
    for (int r = 0; r < ranks; ++r) {
      if (load[r] + c >= best) continue;
      // Owners with equal loads lead to the same subtrees: try the first one only.
      bool seen = false;
      for (int q = 0; q < r && !seen; ++q) seen = load[q] == load[r];
      if (seen) continue;
      const double before = load[r];  // restored exactly afterwards
      load[r] = before + c;
      cur[k] = r;
      dfs(k + 1, std::max(max_load, load[r]), sum_load + c);
      load[r] = before;
      if (aborted || best <= lower) return;
    }
  }
};

}  // namespace

extern "C" int muon_owner_assign(const double* cost, int32_t count, int32_t ranks,
                                 int64_t node_limit, int32_t* owner, double* makespan,
                                 int32_t* optimal) {
  if (count < 0 || ranks < 1 || node_limit < 0) return MUON_EINVAL;
  if (count > 0 && (!cost || !owner)) return MUON_EINVAL;
  for (int32_t i = 0; i < count; ++i)
    if (!std::isfinite(cost[i]) || cost[i] < 0.0) return MUON_EINVAL;
  try {
    // 1. Greedy longest-first.
    std::vector<int> order(static_cast<size_t>(count));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return cost[a] > cost[b]; });
    std::vector<double> load(size_t(ranks), 0.0);
    for (int i : order) {
      int r = 0;
      for (int q = 1; q < ranks; ++q)
        if (load[q] < load[r]) r = q;
      owner[i] = r;
      load[r] += cost[i];
    }
    double best = count > 0 ? *std::max_element(load.begin(), load.end()) : 0.0;
    double total = 0.0, largest = 0.0;
    for (int32_t i = 0; i < count; ++i) {
      total += cost[i];
      largest = std::max(largest, cost[i]);
    }
    const double lower = std::max(largest, total / ranks);
    bool proven = best <= lower;

    // 2. Exact search on small instances.
    if (!proven && count <= kExactMax && node_limit > 0) {
      std::vector<double> sorted(static_cast<size_t>(count));
      for (int k = 0; k < count; ++k) sorted[size_t(k)] = cost[order[size_t(k)]];
      Search s;
      s.cost = &sorted;
      s.ranks = ranks;
      s.node_limit = node_limit;
      s.best = best;
      s.lower = lower;
      s.load.assign(size_t(ranks), 0.0);
      s.cur.assign(size_t(count), 0);
      s.rem.assign(size_t(count) + 1, 0.0);
      for (int k = count - 1; k >= 0; --k) s.rem[size_t(k)] = s.rem[size_t(k) + 1] + sorted[size_t(k)];
      s.dfs(0, 0.0, 0.0);
      if (!s.best_owner.empty()) {
        for (int k = 0; k < count; ++k) owner[order[size_t(k)]] = s.best_owner[size_t(k)];
        best = s.best;
      }
      proven = !s.aborted || s.best <= lower;
    }
    if (makespan) *makespan = best;
    if (optimal) *optimal = proven ? 1 : 0;
    return MUON_OK;
  } catch (...) {
    return MUON_EINVAL;
  }
}
