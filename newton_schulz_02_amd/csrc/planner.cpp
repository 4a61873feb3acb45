// Host planner of muon_step (see planner.h).
//
// Method (DMuon summary §2.2): for X (m x n, m <= n) normalised to X0, the Gram iteration
// keeps G = X X^T and, per step, P = aI + bG + cG^2, G <- P G P, Q <- P Q; the result is
// O = Q X0.  A restart before step k folds Q into X (X <- Q X), re-forms G = X X^T and
// restarts Q, which is exact in real arithmetic.  Every m x m product is a polynomial in
// G0, hence symmetric, so it is computed on lower-triangle tiles and mirrored on store.
// Matrices are sorted into shape buckets and same-level ops of a bucket share one launch
// (DMuon summary §2.2, batching of similar shapes).
#include "planner.h"
#include "tile_order.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <sstream>

namespace muon {

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int kNone = INT_MIN;

int64_t tri_tiles_of(int64_t m) {
  const int64_t t = ceil_div(m, kTile);
  return t * (t + 1) / 2;
}
int64_t full_tiles_of(int64_t rows, int64_t cols) {
  return ceil_div(rows, kTile) * ceil_div(cols, kTile);
}
int fixed_buf(int b) { return -(1 + b); }

// One op of a matrix schedule with symbolic operands: a value v >= 0 is a Gram iterate,
// fixed_buf(b) is a fixed buffer, kNone is unused.
struct SOp {
  int8_t kind;
  int a, b, c, c2, e;
  int8_t alpha, tri;
  int level;
};

// Build the op schedule of one matrix (see the file comment).  Returns the number of
// Gram values created.
int schedule(int steps, uint32_t restarts, bool tall, std::vector<SOp>* ops) {
  int nv = 0;
  int level = 0;
  int xt = fixed_buf(kXtIn);
  int xr = fixed_buf(kXrIn);
  int8_t xscale = kAlphaS;
  int Q = -1;
  if (steps == 0) {
    Q = nv++;
    ops->push_back({kOpIdent, kNone, kNone, Q, kNone, kNone, kAlphaOne, 1, 0});
    level = 1;
  } else {
    int G = nv++;
    ops->push_back({kOpSyrk, xr, xr, G, kNone, kNone, kAlphaS2, 1, level});
    level = 1;
    for (int k = 0; k < steps; ++k) {
      if (((restarts >> k) & 1u) && Q >= 0) {
        const int xr2 = fixed_buf(kXrWs);
        const int xt2 = fixed_buf(xt == fixed_buf(kXtWs0) ? kXtWs1 : kXtWs0);
        ops->push_back({kOpXform, Q, xt, xr2, xt2, kNone, xscale, 0, level});
        ++level;
        xr = xr2;
        xt = xt2;
        xscale = kAlphaOne;
        G = nv++;
        ops->push_back({kOpSyrk, xr, xr, G, kNone, kNone, kAlphaOne, 1, level});
        ++level;
        Q = -1;
      }
      const int P = nv++;
      ops->push_back({kOpPoly, G, G, P, kNone, G, kAlphaOne, 1, level});
      ++level;
      bool emitted = false;
      if (Q < 0) {
        Q = P;
      } else {
        const int Qn = nv++;
        ops->push_back({kOpProd, P, Q, Qn, kNone, kNone, kAlphaOne, 1, level});
        Q = Qn;
        emitted = true;
      }
      const bool restart_next = (k + 1 < steps) && ((restarts >> (k + 1)) & 1u);
      if (k + 1 < steps && !restart_next) {
        const int T = nv++;
        ops->push_back({kOpProd, P, G, T, kNone, kNone, kAlphaOne, 1, level});
        const int G2 = nv++;
        ops->push_back({kOpProd, T, P, G2, kNone, kNone, kAlphaOne, 1, level + 1});
        G = G2;
        level += 2;
      } else if (emitted) {
        level += 1;
      }
    }
  }
  if (!tall)
    ops->push_back({kOpUpdate, Q, xt, fixed_buf(kW), kNone, kNone, xscale, 0, level});
  else
    ops->push_back({kOpUpdate, xt, Q, fixed_buf(kW), kNone, kNone, xscale, 0, level});
  return nv;
}

// Assign Gram values to the kSlots buffers: a value takes the lowest slot whose previous
// value was last read at an earlier level (launches of one stream run in order).
bool assign_slots(std::vector<SOp>& ops, int nv, std::vector<PlanOp>* out) {
  std::vector<int> last(nv, -1), slot(nv, -1);
  for (const SOp& o : ops) {
    for (int v : {o.a, o.b, o.e})
      if (v >= 0) last[v] = std::max(last[v], o.level);
  }
  int busy_until[kSlots];
  for (int& b : busy_until) b = -1;
  std::stable_sort(ops.begin(), ops.end(),
                   [](const SOp& x, const SOp& y) { return x.level < y.level; });
  for (const SOp& o : ops) {
    if (o.c >= 0) {
      int s = -1;
      for (int i = 0; i < kSlots; ++i) {
        if (busy_until[i] < o.level) {
          s = i;
          break;
        }
      }
      if (s < 0) return false;
      slot[o.c] = s;
      busy_until[s] = std::max(last[o.c], o.level);
    }
  }
  auto map = [&](int v) -> int8_t {
    if (v == kNone) return -1;
    if (v >= 0) return int8_t(kSlot0 + slot[v]);
    return int8_t(-v - 1);
  };
  for (const SOp& o : ops)
    out->push_back({o.kind, map(o.a), map(o.b), map(o.c), map(o.c2), map(o.e), o.alpha, o.tri,
                    o.level});
  return true;
}

double op_flops(const PlanOp& o, int64_t m, int64_t n) {
  const double M = double(m), N = double(n);
  switch (o.kind) {
    case kOpSyrk: return M * (M + 1) * N;
    case kOpPoly:
    case kOpProd: return M * (M + 1) * M;
    case kOpXform:
    case kOpUpdate: return 2.0 * M * M * N;
    default: return 0.0;
  }
}

// K-steps of one tile of op o on matrix p: the contraction (n for the Gram formation, m for
// every other product, none for the identity) padded to kKPad, over the elements one
// 128-byte operand row of a stage holds.
int op_ksteps(const PlanOp& o, const PlanMat& p) {
  if (o.kind == kOpIdent) return 0;
  const int64_t len = round_up(o.kind == kOpSyrk ? p.n : p.m, kKPad);
  return int(len * int64_t(p.gsize) / 128);
}

int64_t align_up(int64_t x) { return round_up(x, kAlign); }

}  // namespace

// Gram dtype (see planner.h).
int gram_dtype(int dtype, int64_t m) { return (dtype == kBF16 && m <= kF32GramMaxM) ? int(kF32) : dtype; }

namespace {

struct Span {
  uintptr_t lo, hi;
  int mat;
  bool output;
};

}  // namespace

// Automatic restart set: near-square matrices (n < 1.5 m) re-anchor before every step from
// the third on; others never.  With bf16 iterates stored symmetric, the Gram iterate of a
// near-square matrix loses its small eigenvalues (its smallest singular values are far
// below the largest); folding Q back into X keeps them.  For m = n a restart costs no
// extra flops: the re-anchor (2 m^2 n) and the new Gram matrix (m^2 n) replace three
// m x m products.
uint32_t resolve_restarts(uint32_t mask, int64_t m, int64_t n, int steps) {
  if (mask == MUON_RESTART_AUTO) mask = (2 * n < 3 * m) ? ~3u : 0u;
  const uint32_t valid = steps >= 32 ? 0xFFFFFFFFu : ((1u << steps) - 1u);
  return mask & valid & ~1u;
}

int build_plan(const muon_matrix* mats, int32_t count, const muon_hparams* hp, Plan* plan,
               std::string* err, const CfgChooser* choose) {
  *plan = Plan();
  if (count < 0) {
    *err = "count is negative";
    return MUON_EINVAL;
  }
  if (!hp) {
    *err = "hparams is NULL";
    return MUON_EINVAL;
  }
  if (count > 0 && !mats) {
    *err = "mats is NULL";
    return MUON_EINVAL;
  }
  const float fs[] = {hp->lr, hp->beta, hp->ns_a, hp->ns_b, hp->ns_c, hp->eps};
  for (float f : fs) {
    if (!std::isfinite(f)) {
      *err = "non-finite hyperparameter";
      return MUON_EINVAL;
    }
  }
  if (hp->eps < 0.0f) {
    *err = "eps is negative";
    return MUON_EINVAL;
  }
  if (hp->ns_steps < 0 || hp->ns_steps > 31) {
    *err = "ns_steps outside [0, 31]";
    return MUON_EINVAL;
  }
  std::vector<Span> spans;
  for (int i = 0; i < count; ++i) {
    const muon_matrix& x = mats[i];
    char buf[160];
    if (!x.param || !x.grad || !x.momentum) {
      snprintf(buf, sizeof buf, "matrix %d: NULL pointer", i);
      *err = buf;
      return MUON_EINVAL;
    }
    if (x.rows < 1 || x.cols < 1 || x.rows > kMaxDim || x.cols > kMaxDim) {
      snprintf(buf, sizeof buf, "matrix %d: rows/cols %lld x %lld outside [1, %lld]", i,
               (long long)x.rows, (long long)x.cols, (long long)kMaxDim);
      *err = buf;
      return MUON_EINVAL;
    }
    if (x.dtype != MUON_BF16 && x.dtype != MUON_F32) {
      snprintf(buf, sizeof buf, "matrix %d: unknown dtype %d", i, x.dtype);
      *err = buf;
      return MUON_EINVAL;
    }
    if (x.reserved != 0) {
      snprintf(buf, sizeof buf, "matrix %d: reserved field must be 0", i);
      *err = buf;
      return MUON_EINVAL;
    }
    const uintptr_t es = x.dtype == MUON_BF16 ? 2 : 4;
    if ((uintptr_t)x.param % es || (uintptr_t)x.grad % es || (uintptr_t)x.momentum % es) {
      snprintf(buf, sizeof buf, "matrix %d: pointer not aligned to its element size", i);
      *err = buf;
      return MUON_EINVAL;
    }
    const uintptr_t bytes = uintptr_t(x.rows) * uintptr_t(x.cols) * es;
    spans.push_back({(uintptr_t)x.param, (uintptr_t)x.param + bytes, i, true});
    spans.push_back({(uintptr_t)x.momentum, (uintptr_t)x.momentum + bytes, i, true});
    spans.push_back({(uintptr_t)x.grad, (uintptr_t)x.grad + bytes, i, false});
  }
  // Aliasing: no output may overlap another output or any gradient.
  std::sort(spans.begin(), spans.end(),
            [](const Span& a, const Span& b) { return a.lo < b.lo; });
  {
    // Sweep: track the furthest-reaching output and gradient seen so far.
    uintptr_t out_hi = 0, grad_hi = 0;
    int out_mat = -1, grad_mat = -1;
    for (const Span& s : spans) {
      const bool hits_out = s.lo < out_hi;
      const bool hits_grad = s.output && s.lo < grad_hi;
      if (hits_out || hits_grad) {
        char buf[160];
        snprintf(buf, sizeof buf, "matrix %d: buffer overlaps a %s of matrix %d", s.mat,
                 hits_out ? "param/momentum" : "grad", hits_out ? out_mat : grad_mat);
        *err = buf;
        return MUON_EALIAS;
      }
      if (s.output) {
        if (s.hi > out_hi) out_hi = s.hi, out_mat = s.mat;
      } else if (s.hi > grad_hi) {
        grad_hi = s.hi, grad_mat = s.mat;
      }
    }
  }

  const int steps = hp->ns_steps;
  plan->mats.resize(count);
  for (int i = 0; i < count; ++i) {
    PlanMat& p = plan->mats[i];
    const muon_matrix& x = mats[i];
    p.orig = i;
    p.r = x.rows;
    p.c = x.cols;
    p.tall = x.rows > x.cols;
    p.m = std::min(p.r, p.c);
    p.n = std::max(p.r, p.c);
    p.mp = round_up(p.m, kKPad);
    p.np = round_up(p.n, kKPad);
    p.dtype = x.dtype;
    p.esize = x.dtype == MUON_BF16 ? 2 : 4;
    p.gdtype = gram_dtype(p.dtype, p.m);
    p.gsize = p.gdtype == kBF16 ? 2 : 4;
    p.restarts = resolve_restarts(hp->restart_mask, p.m, p.n, steps);
  }
  std::stable_sort(plan->mats.begin(), plan->mats.end(), [](const PlanMat& a, const PlanMat& b) {
    if (a.gdtype != b.gdtype) return a.gdtype < b.gdtype;
    if (a.dtype != b.dtype) return a.dtype < b.dtype;
    if (a.restarts != b.restarts) return a.restarts < b.restarts;
    if (a.tall != b.tall) return a.tall < b.tall;
    // Larger shapes first: inside a launch the tiles then run longest contraction first.
    if (a.m != b.m) return a.m > b.m;
    if (a.n != b.n) return a.n > b.n;
    return a.orig < b.orig;
  });

  // Schedules and tile counts.
  int max_level = -1;
  int64_t tri = 0, full = 0, mom = 0, wide[3] = {0, 0, 0}, small[2] = {0, 0};
  for (PlanMat& p : plan->mats) {
    std::vector<SOp> sops;
    const int nv = schedule(steps, p.restarts, p.tall, &sops);
    if (!assign_slots(sops, nv, &p.ops)) {
      *err = "internal: Gram slot assignment failed";
      return MUON_EINVAL;
    }
    for (const PlanOp& o : p.ops) {
      max_level = std::max(max_level, o.level);
      p.flops += op_flops(o, p.m, p.n);
    }
    p.tri_tiles = tri_tiles_of(p.m);
    p.full_tiles = full_tiles_of(p.m, p.n);
    p.wide_tiles[0] = sym_tiles(int(p.m), kWideM, kWideN);
    p.wide_tiles[1] = ceil_div(p.m, kWideM) * ceil_div(p.n, kWideN);
    p.wide_tiles[2] = ceil_div(p.n, kWideM) * ceil_div(p.m, kWideN);
    {
      const int64_t ts = ceil_div(p.m, kSmallTile);
      p.small_tiles[0] = ts * (ts + 1) / 2;
      p.small_tiles[1] = ts * ceil_div(p.n, kSmallTile);
    }
    {  // largest operand, with a tile's overhang of rows, below 2^31 bytes
      const int64_t big = std::max(p.m, p.n);
      p.wide_ok = (big + kWideN) * round_up(big, kKPad) * int64_t(p.gsize) < (int64_t(1) << 31);
      p.buf_ok = big * round_up(big, kKPad) * int64_t(p.gsize) < (int64_t(1) << 31);
    }
    // Momentum tiles cover the extents rounded up to kKPad, so that the zero padding of the
    // row and transposed copies (leading dimensions rounded to kKPad) is written too.
    p.mom_tiles_c = round_up(p.c, kKPad) / kEwTile;
    p.mom_tiles_r = round_up(p.r, kKPad) / kEwTile;
    p.mom_tiles = p.mom_tiles_r * p.mom_tiles_c;
    p.tri_prefix = tri;
    p.full_prefix = full;
    for (int k = 0; k < 3; ++k) {
      p.wide_prefix[k] = wide[k];
      wide[k] += p.wide_tiles[k];
    }
    for (int k = 0; k < 2; ++k) {
      p.small_prefix[k] = small[k];
      small[k] += p.small_tiles[k];
    }
    p.mom_prefix = mom;
    tri += p.tri_tiles;
    full += p.full_tiles;
    mom += p.mom_tiles;
    // Compulsory HBM bytes of the elementwise phase: read G and M, write M'.
    p.bytes = 3.0 * double(p.r) * double(p.c) * double(p.esize);
    plan->flops += p.flops;
    plan->bytes += p.bytes;
  }
  if (tri > INT32_MAX || full > INT32_MAX || mom > INT32_MAX || wide[0] > INT32_MAX ||
      wide[1] > INT32_MAX || wide[2] > INT32_MAX || small[0] > INT32_MAX || small[1] > INT32_MAX) {
    *err = "too many tiles for one call";
    return MUON_EINVAL;
  }
  plan->levels = max_level + 1;
  plan->total_mom_tiles = mom;

  // Workspace layout: the status word, then the descriptors.
  int64_t off = kStatusBytes;
  plan->desc_off = off;
  off = align_up(off + int64_t(count) * int64_t(sizeof(MatDesc)));
  plan->scale_off = off;
  off = align_up(off + int64_t(count) * 4);
  plan->partial_off = off;
  off = align_up(off + mom * 4);
  plan->split_cnt_off = off;
  plan->split_cnt_n = 2 * kMaxUnits;
  off = align_up(off + int64_t(plan->split_cnt_n) * 4);
  // The partial-sum slots of the split go last, sized once the launches are known.
  for (PlanMat& p : plan->mats) {
    for (int64_t& o : p.off) o = -1;
    const int64_t es = int64_t(p.gsize);  // Gram iterates and X forms hold the Gram dtype
    for (int s = 0; s < kSlots; ++s) {
      p.off[kSlot0 + s] = off;
      off = align_up(off + p.m * p.mp * es);
    }
    p.off[kXrIn] = off;  // row form copy (m x np), used unless the caller buffer qualifies
    off = align_up(off + p.m * p.np * es);
    p.off[kXtIn] = off;  // transposed form copy (n x mp)
    off = align_up(off + p.n * p.mp * es);
    const int nrestart = __builtin_popcount(p.restarts);
    if (nrestart > 0) {
      p.off[kXrWs] = off;
      off = align_up(off + p.m * p.np * es);
      p.off[kXtWs0] = off;
      off = align_up(off + p.n * p.mp * es);
    }
    if (nrestart > 1) {
      p.off[kXtWs1] = off;
      off = align_up(off + p.n * p.mp * es);
    }
  }
  int64_t ws_end = off;

  // Launches: momentum per run of one input dtype, the norm, then per level and Gram dtype
  // the grouped GEMMs (the sort keeps both kinds of run contiguous).
  auto runs = [&](auto key) {
    std::vector<std::pair<int, int>> out;  // [first, last)
    for (int i = 0; i < count;) {
      int j = i;
      while (j < count && key(plan->mats[j]) == key(plan->mats[i])) ++j;
      out.push_back({i, j});
      i = j;
    }
    return out;
  };
  const auto mom_ranges = runs([](const PlanMat& p) { return p.dtype; });
  const auto ranges = runs([](const PlanMat& p) { return p.gdtype; });
  for (auto [f, l] : mom_ranges) {
    PlanLaunch L;
    L.kind = kLaunchMomentum;
    L.dtype = plan->mats[f].dtype;
    L.first = f;
    L.last = l;
    for (int i = f; i < l; ++i) {
      L.tiles += plan->mats[i].mom_tiles;
      L.bytes += plan->mats[i].bytes;
    }
    plan->launches.push_back(L);
  }
  if (count > 0) {
    PlanLaunch L;
    L.kind = kLaunchNorm;
    L.tiles = count;
    plan->launches.push_back(L);
  }
  for (int lev = 0; lev <= max_level; ++lev) {
    for (auto [f, l] : ranges) {
      struct G {
        PlanOp op;
        int first, last;
      };
      std::vector<G> groups;
      for (int i = f; i < l; ++i) {
        for (const PlanOp& o : plan->mats[i].ops) {
          if (o.level != lev) continue;
          bool joined = false;
          for (G& g : groups) {
            if (g.last == i && g.op.same_sig(o)) {
              g.last = i + 1;
              joined = true;
              break;
            }
          }
          if (!joined) groups.push_back({o, i, i + 1});
        }
      }
      // Longest tiles first (per-tile cost grows with the contraction length), so a launch
      // does not end on a few long tiles.
      auto tile_k = [&](const G& g) {
        const PlanMat& p = plan->mats[g.first];
        return g.op.kind == kOpSyrk ? p.n : p.m;
      };
      std::stable_sort(groups.begin(), groups.end(),
                       [&](const G& x, const G& y) { return tile_k(x) > tile_k(y); });
      for (size_t g0 = 0; g0 < groups.size(); g0 += kMaxGroups) {
        PlanLaunch L;
        // Per tile shape, the end of each matrix's run of tiles and its k-steps.
        std::vector<std::pair<int64_t, int>> tile_runs[kNumShapes];
        L.kind = kLaunchGemm;
        L.dtype = plan->mats[f].gdtype;
        L.level = lev;
        std::ostringstream sig;
        sig << (L.dtype == kBF16 ? "bf16" : "f32");
        for (size_t gi = g0; gi < std::min(groups.size(), g0 + kMaxGroups); ++gi) {
          const G& g = groups[gi];
          const PlanMat& p0 = plan->mats[g.first];
          GroupArg a;
          a.first = g.first;
          a.last = g.last;
          a.kind = g.op.kind;
          a.a = g.op.a;
          a.b = g.op.b;
          a.c = g.op.c;
          a.c2 = g.op.c2;
          a.e = g.op.e;
          a.alpha = g.op.alpha;
          a.tri = g.op.tri;
          a.nm = (g.op.kind == kOpUpdate && p0.tall) ? 1 : 0;  // W is n x m
          for (int i = g.first; i < g.last; ++i) {
            L.wide_ok = L.wide_ok && plan->mats[i].wide_ok;
            L.buf_ok = L.buf_ok && plan->mats[i].buf_ok;
          }
          for (int sh = 0; sh < kNumShapes; ++sh) {
            a.tile_begin = int32_t(L.tiles_cfg[sh]);
            int64_t tpm = -1;
            for (int i = g.first; i < g.last; ++i) {
              const PlanMat& p = plan->mats[i];
              const int64_t nt = sh == kCfgSquare  ? (g.op.tri ? p.tri_tiles : p.full_tiles)
                                 : sh == kShapeSmall ? p.small_tiles[g.op.tri ? 0 : 1]
                                                     : p.wide_tiles[g.op.tri ? 0 : (a.nm ? 2 : 1)];
              tile_runs[sh].push_back({L.tiles_cfg[sh] + nt, op_ksteps(g.op, p)});
              L.tiles_cfg[sh] += nt;
              tpm = (tpm < 0 || tpm == nt) ? nt : 0;
            }
            a.tpm = int32_t(std::max<int64_t>(tpm, 0));
            L.groups_cfg[sh].push_back(a);
          }
          for (int i = g.first; i < g.last; ++i) L.flops += op_flops(g.op, plan->mats[i].m, plan->mats[i].n);
          sig << "|" << int(g.op.kind) << ":" << int(g.op.tri) << ":" << int(a.nm);
          for (int i = g.first; i < g.last;) {  // shapes of the group, run-length encoded
            int j = i;
            while (j < g.last && plan->mats[j].m == plan->mats[i].m && plan->mats[j].n == plan->mats[i].n) ++j;
            sig << ":" << plan->mats[i].m << "x" << plan->mats[i].n << "*" << (j - i);
            i = j;
          }
        }
        for (int sh = 0; sh < kNumShapes; ++sh) {
          if (L.tiles_cfg[sh] > INT32_MAX) {
            *err = "too many tiles in one launch";
            return MUON_EINVAL;
          }
          // Fewest k-steps among the tiles a tail split may cut (the last kMaxUnits).
          const int64_t from = std::max<int64_t>(0, L.tiles_cfg[sh] - kMaxUnits);
          int64_t begin = 0;
          int kmin = INT_MAX;
          for (const auto& [end, ks] : tile_runs[sh]) {
            if (end > from && end > begin) kmin = std::min(kmin, ks);
            begin = end;
          }
          L.kmin_cfg[sh] = kmin == INT_MAX ? 0 : kmin;
        }
        L.signature = sig.str();
        L.cfg = choose ? (*choose)(L.signature) : -1;
        if (L.cfg < 0) L.cfg = default_cfg(L.tiles_cfg[kCfgSquare]);
        plan->launches.push_back(L);
      }
    }
  }
  // Partial-sum slots of the tail split: enough for any unit count up to kMaxUnits (a tail
  // of R < units tiles has at most 2 R pieces in the uneven mode and at most units, and
  // kMaxPieces per tile, in the equal mode).
  int64_t slots = 0;
  for (const PlanLaunch& L : plan->launches) {
    if (L.kind != kLaunchGemm) continue;
    for (int sh = 0; sh < kNumShapes; ++sh) {
      if (L.kmin_cfg[sh] / kSplitUnit < 4) continue;
      const int64_t T = L.tiles_cfg[sh];
      slots = std::max(slots, std::max(std::min<int64_t>(2 * T, 2 * kMaxUnits),
                                       std::min<int64_t>(kMaxPieces * T, kMaxUnits)));
    }
  }
  plan->split_slots = slots;
  plan->split_slot_off = ws_end;
  plan->ws_bytes = size_t(align_up(ws_end + slots * kSlotFloats * 4));
  plan_splits(plan, kMaxUnits);
  return MUON_OK;
}

void plan_splits(Plan* plan, int units) {
  units = std::max(1, std::min(units, kMaxUnits));
  plan->units = units;
  for (PlanLaunch& L : plan->launches) {
    if (L.kind != kLaunchGemm) continue;
    for (int sh = 0; sh < kNumShapes; ++sh)
      L.split_cfg[sh] = plan_split(int(L.tiles_cfg[sh]), units, L.kmin_cfg[sh], kSplitUnit);
    // The chosen configuration, where it applies: the 256 x 384 tiles only when every
    // operand fits their 32-bit offsets, the split only when the launch has a tail to cut.
    int cfg = L.cfg;
    if (cfg < 0 || cfg >= kNumCfg) cfg = kCfgSquare;
    if (cfg_shape(cfg) == kCfgWide && !L.wide_ok) cfg &= ~1;
    // Long fp32 contractions always run split (accuracy: see kF32SplitMinK); the deep
    // pipeline and the small tiles have no split, so such a launch runs the 256 x 256 split.
    if (L.dtype == kF32 && int64_t(L.kmin_cfg[cfg_shape(cfg)]) * 32 >= kF32SplitMinK)
      cfg = (cfg_deep(cfg) || cfg == kCfgSmall) ? int(kCfgSquareSplit) : (cfg | 2);
    if (cfg_split(cfg) && L.split_cfg[cfg_shape(cfg)].mode == kSplitNone) cfg &= ~2;
    L.cfg = cfg;
    const int sh = cfg_shape(cfg);
    L.groups = L.groups_cfg[sh];
    L.tiles = L.tiles_cfg[sh];
    const SplitPlan& sp = L.split_cfg[sh];
    L.grid = cfg_split(cfg) ? int64_t(sp.dp_tiles) + sp.tail_wgs : L.tiles;
  }
}

void fill_descs(const Plan& plan, const muon_matrix* mats, const muon_hparams* hp, char* ws,
                std::vector<MatDesc>* out) {
  out->assign(plan.mats.size(), MatDesc());
  for (size_t i = 0; i < plan.mats.size(); ++i) {
    const PlanMat& p = plan.mats[i];
    const muon_matrix& x = mats[p.orig];
    MatDesc& d = (*out)[i];
    std::memset(&d, 0, sizeof d);
    auto at = [&](int id) -> void* { return p.off[id] >= 0 ? ws + p.off[id] : nullptr; };
    const int64_t es = int64_t(p.esize);
    d.grad = x.grad;
    d.mom = x.momentum;
    d.rows = int32_t(p.r);
    d.cols = int32_t(p.c);
    d.vec = ((uintptr_t)x.grad % 16 == 0 && (uintptr_t)x.momentum % 16 == 0 &&
             (p.c * es) % 16 == 0)
                ? 1
                : 0;
    d.wvec = ((uintptr_t)x.param % 16 == 0 && (p.c * es) % 16 == 0) ? 1 : 0;
    // The caller's momentum can serve as a form of X when it has the Gram dtype, a 128-multiple
    // leading dimension and 16-byte alignment.
    const bool caller_ok = p.gdtype == p.dtype && (p.c % kKPad == 0) && ((uintptr_t)x.momentum % 16 == 0);
    d.gram_f32 = (p.gdtype == kF32 && p.dtype == kBF16) ? 1 : 0;
    for (int s = 0; s < kSlots; ++s)
      d.buf[kSlot0 + s] = {at(kSlot0 + s), p.mp, int32_t(p.m), int32_t(p.mp)};
    const BufDesc row_ws = {at(kXrIn), p.np, int32_t(p.m), int32_t(p.np)};
    const BufDesc t_ws = {at(kXtIn), p.mp, int32_t(p.n), int32_t(p.mp)};
    // Leading dimensions of the copies the momentum kernel writes: row form (m x np) and
    // transposed form (n x mp) of X.
    d.copy_ld = p.tall ? t_ws.ld : row_ws.ld;
    d.trans_ld = p.tall ? row_ws.ld : t_ws.ld;
    if (!p.tall) {
      // X = M' (m = rows): row form is M' itself or its padded copy; X^T is the transpose.
      if (caller_ok) {
        d.buf[kXrIn] = {x.momentum, p.c, int32_t(p.m), int32_t(p.c)};
        d.copy_out = nullptr;
      } else {
        d.buf[kXrIn] = row_ws;
        d.copy_out = row_ws.ptr;
      }
      d.buf[kXtIn] = t_ws;
      d.trans_out = t_ws.ptr;
    } else {
      // X = M'^T (m = cols): row form is the transpose; X^T is M' itself or its copy.
      d.buf[kXrIn] = row_ws;
      d.trans_out = row_ws.ptr;
      if (caller_ok) {
        d.buf[kXtIn] = {x.momentum, p.c, int32_t(p.n), int32_t(p.c)};
        d.copy_out = nullptr;
      } else {
        d.buf[kXtIn] = t_ws;
        d.copy_out = t_ws.ptr;
      }
    }
    d.buf[kXrWs] = {at(kXrWs), p.np, int32_t(p.m), int32_t(p.np)};
    d.buf[kXtWs0] = {at(kXtWs0), p.mp, int32_t(p.n), int32_t(p.mp)};
    d.buf[kXtWs1] = {at(kXtWs1), p.mp, int32_t(p.n), int32_t(p.mp)};
    d.buf[kW] = {x.param, p.c, int32_t(p.r), 0};
    d.mom_prefix = int32_t(p.mom_prefix);
    d.mom_tiles_c = int32_t(p.mom_tiles_c);
    d.mom_tiles_r = int32_t(p.mom_tiles_r);
    d.tri_prefix = int32_t(p.tri_prefix);
    d.full_prefix = int32_t(p.full_prefix);
    for (int k = 0; k < 3; ++k) d.wide_prefix[k] = int32_t(p.wide_prefix[k]);
    for (int k = 0; k < 2; ++k) d.small_prefix[k] = int32_t(p.small_prefix[k]);
    d.eta = float(double(hp->lr) * std::sqrt(std::max(1.0, double(p.r) / double(p.c))));
  }
}

std::string describe_plan(const Plan& plan) {
  static const char* kKind[] = {"syrk", "poly", "prod", "xform", "update", "ident", "affine"};
  std::ostringstream os;
  os.precision(17);
  os << "{\"count\":" << plan.mats.size() << ",\"workspace\":" << plan.ws_bytes
     << ",\"levels\":" << plan.levels << ",\"flops\":" << plan.flops
     << ",\"bytes\":" << plan.bytes << ",\"units\":" << plan.units
     << ",\"desc_off\":" << plan.desc_off << ",\"scale_off\":" << plan.scale_off
     << ",\"partial_off\":" << plan.partial_off << ",\"mom_tiles\":" << plan.total_mom_tiles
     << ",\"split_cnt_off\":" << plan.split_cnt_off << ",\"split_cnt_n\":" << plan.split_cnt_n
     << ",\"split_slot_off\":" << plan.split_slot_off
     << ",\"split_slots\":" << plan.split_slots << ",\"matrices\":[";
  for (size_t i = 0; i < plan.mats.size(); ++i) {
    const PlanMat& p = plan.mats[i];
    os << (i ? "," : "") << "{\"orig\":" << p.orig << ",\"rows\":" << p.r << ",\"cols\":" << p.c
       << ",\"m\":" << p.m << ",\"n\":" << p.n << ",\"tall\":" << (p.tall ? "true" : "false")
       << ",\"dtype\":" << p.dtype << ",\"gram_dtype\":" << p.gdtype << ",\"restarts\":" << p.restarts
       << ",\"flops\":" << p.flops << ",\"regions\":[";
    {  // workspace byte ranges [offset, bytes] of the matrix's own buffers
      const int64_t es = int64_t(p.gsize);
      bool first = true;
      for (int b = 0; b < kNumBuf; ++b) {
        if (p.off[b] < 0) continue;
        const int64_t bytes = b < kSlot0 + kSlots ? p.m * p.mp * es
                              : (b == kXrIn || b == kXrWs) ? p.m * p.np * es : p.n * p.mp * es;
        os << (first ? "" : ",") << "[" << p.off[b] << "," << bytes << "]";
        first = false;
      }
    }
    os << "],\"ops\":[";
    for (size_t j = 0; j < p.ops.size(); ++j) {
      const PlanOp& o = p.ops[j];
      os << (j ? "," : "") << "{\"kind\":\"" << kKind[int(o.kind)] << "\",\"level\":" << o.level
         << ",\"a\":" << int(o.a) << ",\"b\":" << int(o.b) << ",\"c\":" << int(o.c)
         << ",\"c2\":" << int(o.c2) << ",\"e\":" << int(o.e) << ",\"alpha\":" << int(o.alpha)
         << "}";
    }
    os << "]}";
  }
  os << "],\"launches\":[";
  static const char* kLaunch[] = {"momentum", "norm", "gemm", "copy_in", "copy_out"};
  for (size_t i = 0; i < plan.launches.size(); ++i) {
    const PlanLaunch& L = plan.launches[i];
    os << (i ? "," : "") << "{\"kind\":\"" << kLaunch[L.kind] << "\",\"dtype\":" << L.dtype
       << ",\"level\":" << L.level << ",\"tiles\":" << L.tiles << ",\"cfg\":" << L.cfg
       << ",\"grid\":" << L.grid
       << ",\"tiles_cfg\":[" << L.tiles_cfg[0] << "," << L.tiles_cfg[1] << "," << L.tiles_cfg[2] << "]"
       << ",\"kmin_cfg\":[" << L.kmin_cfg[0] << "," << L.kmin_cfg[1] << "," << L.kmin_cfg[2] << "]"
       << ",\"split_cfg\":[";
    for (int sh = 0; sh < kNumShapes; ++sh) {
      const SplitPlan& sp = L.split_cfg[sh];
      os << (sh ? "," : "") << "{\"mode\":" << sp.mode << ",\"c\":" << sp.c << ",\"n\":" << sp.n
         << ",\"dp_tiles\":" << sp.dp_tiles << ",\"tail\":" << sp.tail
         << ",\"tail_wgs\":" << sp.tail_wgs << ",\"slots\":" << sp.slots << "}";
    }
    os << "]"
       << ",\"wide_ok\":" << (L.wide_ok ? "true" : "false")
       << ",\"buf_ok\":" << (L.buf_ok ? "true" : "false")
       << ",\"signature\":\"" << L.signature << "\",\"flops\":" << L.flops
       << ",\"groups\":[";
    for (size_t g = 0; g < L.groups.size(); ++g) {
      const GroupArg& a = L.groups[g];
      os << (g ? "," : "") << "{\"first\":" << a.first << ",\"last\":" << a.last
         << ",\"kind\":\"" << kKind[int(a.kind)] << "\",\"tiles_begin\":" << a.tile_begin
         << ",\"tpm\":" << a.tpm << "}";
    }
    os << "]}";
  }
  os << "]}";
  return os.str();
}

}  // namespace muon
