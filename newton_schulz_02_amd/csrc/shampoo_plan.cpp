// Host planner of shampoo_step (see shampoo_plan.h).
//
// Method (Gupta, Koren and Singer, 2018, for a matrix parameter; the inverse roots by the
// coupled Newton iteration of Guo and Higham, 2006, with p = 4), per statistic S of size m:
//   S <- beta2 S + F F^T            (F = G for the left statistic, G^T for the right one)
//   s = 1 / (||S||_F + eps)         (the momentum kernel's sums of squares and the norm kernel)
//   M_0 = s (S + eps I),  T_0 = (5 I - M_0) / 4
//   for k = 0 .. K-2:  Y_{k+1} = Y_k T_k (Y_1 = T_0),  M_{k+1} = T_k^4 M_k,  T_{k+1} = (5 I - M_{k+1}) / 4
//   root = s^(1/4) Y_{K-1} T_{K-1}  (= s^(1/4) T_0 when K = 1)
// which is the iteration X_0 = nu^(-1/4) I, X_{k+1} = X_k T_k with X_k = nu^(-1/4) Y_k, nu = 1/s.
// T^4 M is formed as (T T)(T T) M: three products, plus Y T.  Every iterate is a polynomial
// in S, so all of them are symmetric and commute; each product is computed on lower-triangle
// tiles and mirrored on store.  Then Z = X_L G (full tiles) and W <- W - lr Z X_R.
#include "shampoo_plan.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <sstream>

namespace muon {

namespace {

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x) { return round_up(x, kAlign); }
int64_t tri_tiles(int64_t m) {
  const int64_t t = ceil_div(m, kTile);
  return t * (t + 1) / 2;
}
int64_t full_tiles(int64_t r, int64_t c) { return ceil_div(r, kTile) * ceil_div(c, kTile); }

constexpr int kFixedX = -2;  // operand code of the accumulation factor (buffer kShX)

// One op of the statistic schedule.  a, b, c, e: values (>= 0), kFixedX or -1 (unused).
struct ROp {
  int8_t kind;
  int a, b, c, e;
  int8_t alpha;
  int level;
};

// Per level: the launch coefficients (pa, pb, pc).
struct LevelCoef {
  float pa, pb, pc;
};

struct Schedule {
  std::vector<ROp> ops;
  std::vector<int> last;       // last level that reads each value (INT_MAX: read after)
  std::vector<LevelCoef> coef; // per level
  int stat = 0, root = 0;      // values of the accumulated statistic and the root
  int levels = 0;
};

Schedule make_schedule(int iters, float beta2, float eps) {
  Schedule sc;
  auto val = [&] {
    sc.last.push_back(-1);
    return int(sc.last.size()) - 1;
  };
  auto use = [&](int v, int lev) { sc.last[size_t(v)] = std::max(sc.last[size_t(v)], lev); };
  const LevelCoef affine_t = {1.25f, -0.25f, 0.0f};
  const LevelCoef none = {0.0f, 0.0f, 0.0f};
  // Level 0: S <- 0 I + beta2 S + 1 F F^T, in place over the copy of the caller's S.
  const int S = val();
  sc.ops.push_back({kOpPoly, kFixedX, kFixedX, S, S, kAlphaOne, 0});
  sc.coef.push_back({0.0f, beta2, 1.0f});
  // Level 1: M_0 = s (eps I + S).
  int M = val();
  sc.ops.push_back({kOpAffine, -1, -1, M, S, kAlphaS, 1});
  use(S, 1);
  sc.coef.push_back({eps, 1.0f, 0.0f});
  // Level 2: T_0 (scaled by s^(1/4) when it is the root).
  int T = val();
  sc.ops.push_back({kOpAffine, -1, -1, T, M, int8_t(iters == 1 ? kAlphaQuarter : kAlphaOne), 2});
  use(M, 2);
  sc.coef.push_back(affine_t);
  int lev = 2;
  int Y = -1;  // Y_k; -1 is the identity
  for (int k = 0; k + 1 < iters; ++k) {
    const int la = lev + 1, lb = lev + 2, lc = lev + 3, ld = lev + 4;
    const int T2 = val();
    sc.ops.push_back({kOpProd, T, T, T2, -1, kAlphaOne, la});
    use(T, la);
    if (Y < 0) {
      Y = T;  // Y_1 = T_0: no product
    } else {
      const int Yn = val();
      sc.ops.push_back({kOpProd, Y, T, Yn, -1, kAlphaOne, la});
      use(Y, la);
      Y = Yn;
    }
    sc.coef.push_back(none);
    const int T4 = val();
    sc.ops.push_back({kOpProd, T2, T2, T4, -1, kAlphaOne, lb});
    use(T2, lb);
    sc.coef.push_back(none);
    const int Mn = val();
    sc.ops.push_back({kOpProd, T4, M, Mn, -1, kAlphaOne, lc});
    use(T4, lc);
    use(M, lc);
    M = Mn;
    sc.coef.push_back(none);
    const int Tn = val();
    sc.ops.push_back({kOpAffine, -1, -1, Tn, M, kAlphaOne, ld});
    use(M, ld);
    T = Tn;
    sc.coef.push_back(affine_t);
    lev = ld;
  }
  int root = T;
  if (iters > 1) {
    root = val();
    ++lev;
    // The last product carries the scale s^(1/4): a SYRK-kind op (alpha A B^T).
    sc.ops.push_back({kOpSyrk, Y, T, root, -1, kAlphaQuarter, lev});
    use(Y, lev);
    use(T, lev);
    sc.coef.push_back(none);
  }
  sc.last[size_t(root)] = INT_MAX;
  sc.stat = S;
  sc.root = root;
  sc.levels = lev + 1;
  return sc;
}

// Slots: a value takes the lowest slot whose previous value was last read at an earlier
// level.  Returns the slot of every value, or an empty vector if kShSlots do not suffice.
std::vector<int> assign(const Schedule& sc, int* used) {
  std::vector<int> slot(sc.last.size(), -1);
  int busy[kShSlots];
  for (int& b : busy) b = -1;
  *used = 0;
  for (const ROp& o : sc.ops) {  // ops are in level order
    int s = -1;
    for (int i = 0; i < kShSlots; ++i)
      if (busy[i] < o.level) {
        s = i;
        break;
      }
    if (s < 0) return {};
    slot[size_t(o.c)] = s;
    busy[s] = std::max(sc.last[size_t(o.c)], o.level);
    *used = std::max(*used, s + 1);
  }
  return slot;
}

struct Span {
  uintptr_t lo, hi;
  int mat;
  bool output;
};

}  // namespace

int build_shampoo_plan(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                       ShampooPlan* sp, std::string* err) {
  *sp = ShampooPlan();
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
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->beta2) || !std::isfinite(hp->eps)) {
    *err = "non-finite hyperparameter";
    return MUON_EINVAL;
  }
  if (hp->beta2 < 0.0f || hp->beta2 > 1.0f) {
    *err = "beta2 outside [0, 1]";
    return MUON_EINVAL;
  }
  if (!(hp->eps > 0.0f)) {
    *err = "eps must be > 0";
    return MUON_EINVAL;
  }
  if (hp->root_iters < 1 || hp->root_iters > kShMaxIters) {
    *err = "root_iters outside [1, 64]";
    return MUON_EINVAL;
  }
  std::vector<Span> spans;
  for (int i = 0; i < count; ++i) {
    const shampoo_matrix& x = mats[i];
    char buf[160];
    if (!x.param || !x.grad || !x.stat_left || !x.stat_right) {
      snprintf(buf, sizeof buf, "matrix %d: NULL pointer", i);
      *err = buf;
      return MUON_EINVAL;
    }
    if (x.rows < 1 || x.cols < 1 || x.rows > kShMaxDim || x.cols > kShMaxDim) {
      snprintf(buf, sizeof buf, "matrix %d: rows/cols %lld x %lld outside [1, %lld]", i,
               (long long)x.rows, (long long)x.cols, (long long)kShMaxDim);
      *err = buf;
      return MUON_EINVAL;
    }
    if (x.dtype != MUON_F32 && x.dtype != MUON_BF16) {
      snprintf(buf, sizeof buf, "matrix %d: unknown dtype %d", i, x.dtype);
      *err = buf;
      return MUON_EINVAL;
    }
    if (x.reserved != 0) {
      snprintf(buf, sizeof buf, "matrix %d: reserved field must be 0", i);
      *err = buf;
      return MUON_EINVAL;
    }
    const uintptr_t ptrs[4] = {(uintptr_t)x.param, (uintptr_t)x.grad, (uintptr_t)x.stat_left,
                               (uintptr_t)x.stat_right};
    const uintptr_t es = x.dtype == MUON_BF16 ? 2 : 4;  // param and grad; statistics are fp32
    if (ptrs[0] % es || ptrs[1] % es || ptrs[2] % 4 || ptrs[3] % 4) {
      snprintf(buf, sizeof buf, "matrix %d: pointer not aligned to its element size", i);
      *err = buf;
      return MUON_EINVAL;
    }
    const uintptr_t r = uintptr_t(x.rows), c = uintptr_t(x.cols);
    spans.push_back({ptrs[0], ptrs[0] + r * c * es, i, true});
    spans.push_back({ptrs[1], ptrs[1] + r * c * es, i, false});
    spans.push_back({ptrs[2], ptrs[2] + r * r * 4, i, true});
    spans.push_back({ptrs[3], ptrs[3] + c * c * 4, i, true});
  }
  // Aliasing: no output may overlap another output or any gradient.
  std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  {
    uintptr_t out_hi = 0, grad_hi = 0;
    int out_mat = -1, grad_mat = -1;
    for (const Span& s : spans) {
      const bool hits_out = s.lo < out_hi;
      const bool hits_grad = s.output && s.lo < grad_hi;
      if (hits_out || hits_grad) {
        char buf[160];
        snprintf(buf, sizeof buf, "matrix %d: buffer overlaps a %s of matrix %d", s.mat,
                 hits_out ? "param/statistic" : "grad", hits_out ? out_mat : grad_mat);
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

  const Schedule sc = make_schedule(hp->root_iters, hp->beta2, hp->eps);
  int used = 0;
  const std::vector<int> slot = assign(sc, &used);
  if (slot.empty()) {
    *err = "internal: statistic slot assignment failed";
    return MUON_EINVAL;
  }
  sp->count = count;
  sp->iters = hp->root_iters;
  sp->slots = used;
  sp->stat_slot = slot[size_t(sc.stat)];
  sp->root_slot = slot[size_t(sc.root)];
  Plan& plan = sp->plan;
  plan.units = kMaxUnits;

  // Entries: the caller's matrices in order, then the statistics largest first.
  struct Stat {
    int64_t m;
    int mat;
    int8_t right;
  };
  std::vector<Stat> stats;
  for (int i = 0; i < count; ++i) {
    stats.push_back({mats[i].rows, i, 0});
    stats.push_back({mats[i].cols, i, 1});
  }
  std::stable_sort(stats.begin(), stats.end(), [](const Stat& a, const Stat& b) { return a.m > b.m; });
  plan.mats.resize(size_t(3) * size_t(count));
  sp->left_entry.assign(size_t(count), -1);
  sp->right_entry.assign(size_t(count), -1);
  int64_t full = 0, tri = 0, mom = 0;
  for (int i = 0; i < count; ++i) {
    PlanMat& p = plan.mats[size_t(i)];
    p.orig = i;
    p.r = mats[i].rows;
    p.c = mats[i].cols;
    p.m = std::min(p.r, p.c);
    p.n = std::max(p.r, p.c);
    p.mp = round_up(p.r, kKPad);  // padded rows (the contraction of X_L G)
    p.np = round_up(p.c, kKPad);  // padded cols (the contraction of Z X_R)
    p.dtype = mats[i].dtype == MUON_BF16 ? int(kBF16) : int(kF32);  // W and G
    p.esize = p.dtype == kBF16 ? 2 : 4;
    p.gdtype = kF32;  // the copies of G, the products and the statistics
    p.gsize = 4;
    p.full_tiles = full_tiles(p.r, p.c);
    p.full_prefix = full;
    full += p.full_tiles;
    p.mom_tiles_c = p.np / kEwTile;
    p.mom_tiles_r = p.mp / kEwTile;
    p.mom_tiles = p.mom_tiles_r * p.mom_tiles_c;
    p.mom_prefix = mom;
    mom += p.mom_tiles;
    // Contractions: G G^T over cols (tri, rows), G^T G over rows (tri, cols), X_L G over rows,
    // Z X_R over cols.
    p.flops = double(p.r) * double(p.r + 1) * double(p.c) + double(p.c) * double(p.c + 1) * double(p.r) +
              2.0 * double(p.r) * double(p.r) * double(p.c) + 2.0 * double(p.r) * double(p.c) * double(p.c);
    // Compulsory HBM bytes: read G, read and write W and both statistics.
    p.bytes = 3.0 * double(p.esize) * double(p.r) * double(p.c) +
              4.0 * (2.0 * double(p.r) * double(p.r) + 2.0 * double(p.c) * double(p.c));
    plan.flops += p.flops;
    plan.bytes += p.bytes;
  }
  for (size_t j = 0; j < stats.size(); ++j) {
    const int e = count + int(j);
    PlanMat& p = plan.mats[size_t(e)];
    p.orig = stats[j].mat;
    p.m = p.r = p.c = p.n = stats[j].m;
    p.mp = p.np = round_up(p.m, kKPad);
    p.dtype = p.gdtype = kF32;
    p.esize = p.gsize = 4;
    p.tri_tiles = tri_tiles(p.m);
    p.tri_prefix = tri;
    tri += p.tri_tiles;
    p.mom_tiles_c = p.mp / kEwTile;
    p.mom_tiles_r = p.mp / kEwTile;
    p.mom_tiles = p.mom_tiles_r * p.mom_tiles_c;
    p.mom_prefix = mom;
    mom += p.mom_tiles;
    sp->stat_mat.push_back(stats[j].mat);
    sp->stat_right.push_back(stats[j].right);
    (stats[j].right ? sp->right_entry : sp->left_entry)[size_t(stats[j].mat)] = e;
    // Products of the root: T T, (T T)(T T) and T^4 M per Newton step, the K - 2 products
    // Y T and the last one: 4 (K - 1), each m(m+1)m.
    const int nprod = 4 * (sp->iters - 1);
    p.flops = double(nprod) * double(p.m) * double(p.m + 1) * double(p.m);
    plan.flops += p.flops;
  }
  if (full > INT32_MAX || tri > INT32_MAX || mom > INT32_MAX) {
    *err = "too many tiles for one call";
    return MUON_EINVAL;
  }
  plan.total_mom_tiles = mom;
  plan.levels = sc.levels;

  // Workspace: descriptors, scales, partial sums, then per gradient entry G, G^T and Z, per
  // statistic entry its slots.
  int64_t off = kStatusBytes;  // the status word comes first
  const int64_t entries = 3 * int64_t(count);
  plan.desc_off = off;
  off = align_up(off + entries * int64_t(sizeof(MatDesc)));
  plan.scale_off = off;
  off = align_up(off + entries * 4);
  plan.partial_off = off;
  off = align_up(off + mom * 4);
  plan.split_cnt_off = off;  // tail split: 2 counters per tail tile
  plan.split_cnt_n = 2 * kMaxUnits;
  off = align_up(off + int64_t(plan.split_cnt_n) * 4);
  for (int i = 0; i < count; ++i) {
    PlanMat& p = plan.mats[size_t(i)];
    for (int64_t& o : p.off) o = -1;
    p.off[kShG] = off;
    off = align_up(off + p.r * p.np * 4);
    p.off[kShGT] = off;
    off = align_up(off + p.c * p.mp * 4);
    p.off[kShZ] = off;
    off = align_up(off + p.r * p.np * 4);
  }
  for (int64_t e = count; e < entries; ++e) {
    PlanMat& p = plan.mats[size_t(e)];
    for (int64_t& o : p.off) o = -1;
    for (int s = 0; s < sp->slots; ++s) {
      p.off[s] = off;
      off = align_up(off + p.m * p.mp * 4);
    }
  }
  plan.split_slot_off = off;  // the partial-sum slots go last, sized once the launches are known
  plan.split_slots = 0;
  plan.ws_bytes = size_t(off);
  if (count == 0) return MUON_OK;

  // Launches.
  auto gemm = [&](int first, int last, int level, const LevelCoef& cf) {
    PlanLaunch L;
    L.kind = kLaunchGemm;
    L.dtype = kF32;
    L.level = level;
    L.first = first;
    L.last = last;
    L.cfg = kCfgSquare;
    L.wide_ok = false;
    // Operands: the statistic slots (m x round_up(m)); for a matrix, the copies of G, G^T and
    // X_L G and the roots X_L and X_R it reads from its statistics' slots.
    for (int e = first; e < last; ++e) {
      const PlanMat& p = plan.mats[size_t(e)];
      const int64_t big = e >= count ? p.m * p.mp
                                     : std::max({p.r * p.np, p.c * p.mp, p.r * p.mp, p.c * p.np});
      L.buf_ok = L.buf_ok && big * 4 < (int64_t(1) << 31);
    }
    L.own_coef = true;
    L.pa = cf.pa;
    L.pb = cf.pb;
    L.pc = cf.pc;
    return L;
  };
  auto add_group = [&](PlanLaunch& L, GroupArg a) {
    a.first = L.first;
    a.last = L.last;
    a.tile_begin = int32_t(L.tiles_cfg[0]);
    int64_t tpm = -1;
    for (int e = L.first; e < L.last; ++e) {
      const PlanMat& p = plan.mats[size_t(e)];
      const int64_t nt = a.tri ? p.tri_tiles : p.full_tiles;
      L.tiles_cfg[0] += nt;
      tpm = (tpm < 0 || tpm == nt) ? nt : 0;
    }
    a.tpm = int32_t(std::max<int64_t>(tpm, 0));
    L.groups_cfg[0].push_back(a);
  };
  // K-steps of one tile of group a on entry e: the contraction (padded) over 32 fp32 values.
  auto ksteps = [&](const GroupArg& a, int e) -> int {
    const PlanMat& p = plan.mats[size_t(e)];
    if (a.kind == kOpAffine) return 0;
    if (e < count) return int((a.kind == kOpXform ? p.mp : p.np) / 32);  // X_L G over rows, Z X_R over cols
    if (a.kind == kOpPoly) {  // F F^T over the other side of the matrix
      const PlanMat& g = plan.mats[size_t(p.orig)];
      return int((sp->stat_right[size_t(e - count)] ? g.mp : g.np) / 32);
    }
    return int(p.mp / 32);
  };
  auto finish = [&](PlanLaunch& L, const char* what) {
    L.groups = L.groups_cfg[0];
    L.tiles = L.tiles_cfg[0];
    L.grid = L.tiles;
    L.signature = what;
    // Fewest k-steps among the tiles a tail split may cut (the last kMaxUnits).
    const int64_t from = std::max<int64_t>(0, L.tiles - kMaxUnits);
    int64_t end = 0;
    int kmin = INT_MAX;
    for (const GroupArg& a : L.groups_cfg[0])
      for (int e = a.first; e < a.last; ++e) {
        const PlanMat& p = plan.mats[size_t(e)];
        end += a.tri ? p.tri_tiles : p.full_tiles;
        if (end > from) kmin = std::min(kmin, ksteps(a, e));
      }
    L.kmin_cfg[0] = kmin == INT_MAX ? 0 : kmin;
    plan.launches.push_back(L);
  };
  auto code = [&](int v) -> int8_t {
    if (v == kFixedX) return int8_t(kShX);
    if (v < 0) return int8_t(-1);
    return int8_t(slot[size_t(v)]);
  };
  const int sfirst = count, slast = int(entries);
  // Copies of G and G^T in fp32 (the momentum kernel with no momentum buffer), one launch per
  // run of matrices of one dtype.
  for (int f = 0; f < count;) {
    int l = f;
    while (l < count && plan.mats[size_t(l)].dtype == plan.mats[size_t(f)].dtype) ++l;
    PlanLaunch L;
    L.kind = kLaunchMomentum;
    L.dtype = plan.mats[size_t(f)].dtype;
    L.first = f;
    L.last = l;
    for (int i = f; i < l; ++i) {
      const PlanMat& p = plan.mats[size_t(i)];
      L.tiles += p.mom_tiles;
      L.bytes += (double(p.esize) + 8.0) * double(p.r) * double(p.c);
    }
    plan.launches.push_back(L);
    f = l;
  }
  {
    PlanLaunch L;
    L.kind = kLaunchCopyIn;
    L.first = sfirst;
    L.last = slast;
    plan.launches.push_back(L);
  }
  for (int lev = 0; lev < sc.levels; ++lev) {
    PlanLaunch L = gemm(sfirst, slast, lev, sc.coef[size_t(lev)]);
    for (const ROp& o : sc.ops) {
      if (o.level != lev) continue;
      GroupArg a;
      a.kind = o.kind;
      a.a = code(o.a);
      a.b = code(o.b);
      a.c = code(o.c);
      a.c2 = -1;
      a.e = code(o.e);
      a.alpha = o.alpha;
      a.tri = 1;
      a.nm = 0;
      add_group(L, a);
      for (int e = sfirst; e < slast; ++e) {
        const PlanMat& p = plan.mats[size_t(e)];
        const int64_t k = o.kind == kOpPoly ? plan.mats[size_t(p.orig)].c + plan.mats[size_t(p.orig)].r - p.m : p.m;
        if (o.kind != kOpAffine) L.flops += double(p.m) * double(p.m + 1) * double(k);
      }
    }
    finish(L, "shampoo");
    if (lev == 0) {
      // The accumulated statistics go back to the caller, and their Frobenius norms give
      // the scales s (the momentum kernel over the slot, no momentum buffer, then the norm).
      PlanLaunch out;
      out.kind = kLaunchCopyOut;
      out.first = sfirst;
      out.last = slast;
      plan.launches.push_back(out);
      PlanLaunch ms;
      ms.kind = kLaunchMomentum;
      ms.dtype = kF32;
      ms.first = sfirst;
      ms.last = slast;
      for (int e = sfirst; e < slast; ++e) {
        ms.tiles += plan.mats[size_t(e)].mom_tiles;
        ms.bytes += 4.0 * double(plan.mats[size_t(e)].m) * double(plan.mats[size_t(e)].mp);
      }
      plan.launches.push_back(ms);
      PlanLaunch nm;
      nm.kind = kLaunchNorm;
      nm.tiles = entries;
      plan.launches.push_back(nm);
    }
  }
  {  // Z = X_L G: A = X_L (rows x rows), B = G^T (cols x rows), full tiles rows x cols
    PlanLaunch L = gemm(0, count, sc.levels, {0.0f, 0.0f, 0.0f});
    GroupArg a;
    a.kind = kOpXform;
    a.a = kShXL;
    a.b = kShGT;
    a.c = kShZ;
    a.c2 = -1;
    a.e = -1;
    a.alpha = kAlphaOne;
    a.tri = 0;
    a.nm = 0;
    add_group(L, a);
    for (int i = 0; i < count; ++i) {
      const PlanMat& p = plan.mats[size_t(i)];
      L.flops += 2.0 * double(p.r) * double(p.r) * double(p.c);
    }
    finish(L, "shampoo");
  }
  {  // W <- W - lr Z X_R: A = Z (rows x cols), B = X_R (cols x cols)
    PlanLaunch L = gemm(0, count, sc.levels + 1, {0.0f, 0.0f, 0.0f});
    GroupArg a;
    a.kind = kOpUpdate;
    a.a = kShZ;
    a.b = kShXR;
    a.c = kW;
    a.c2 = -1;
    a.e = -1;
    a.alpha = kAlphaOne;
    a.tri = 0;
    a.nm = 0;
    add_group(L, a);
    for (int i = 0; i < count; ++i) {
      const PlanMat& p = plan.mats[size_t(i)];
      L.flops += 2.0 * double(p.r) * double(p.c) * double(p.c);
    }
    finish(L, "shampoo");
  }
  // Partial-sum slots of the tail split, enough for any unit count up to kMaxUnits (as in the
  // Muon plan).  The accumulation (level 0) runs before the norm kernel clears the split
  // counters, so it is never split.
  int64_t slots = 0;
  for (const PlanLaunch& L : plan.launches) {
    if (L.kind != kLaunchGemm) continue;
    if (L.tiles_cfg[0] > INT32_MAX) {
      *err = "too many tiles in one launch";
      return MUON_EINVAL;
    }
    if (L.level == 0 || L.kmin_cfg[0] / kSplitUnit < 4) continue;
    const int64_t T = L.tiles_cfg[0];
    slots = std::max(slots, std::max(std::min<int64_t>(2 * T, 2 * kMaxUnits),
                                     std::min<int64_t>(kMaxPieces * T, kMaxUnits)));
  }
  plan.split_slots = slots;
  plan.ws_bytes = size_t(align_up(int64_t(plan.ws_bytes) + slots * kSlotFloats * 4));
  shampoo_plan_splits(sp, kMaxUnits, -1);
  return MUON_OK;
}

void shampoo_plan_splits(ShampooPlan* sp, int units, int force_cfg) {
  Plan& plan = sp->plan;
  units = std::max(1, std::min(units, kMaxUnits));
  plan.units = units;
  for (PlanLaunch& L : plan.launches) {
    if (L.kind != kLaunchGemm) continue;
    L.split_cfg[0] = L.level == 0 ? SplitPlan() : plan_split(int(L.tiles_cfg[0]), units, L.kmin_cfg[0], kSplitUnit);
    if (L.level == 0) L.split_cfg[0].dp_tiles = int(L.tiles_cfg[0]);
    const bool want = force_cfg < 0 || cfg_split(force_cfg);
    const SplitPlan& s = L.split_cfg[0];
    L.cfg = (want && s.mode != kSplitNone) ? int(kCfgSquareSplit) : int(kCfgSquare);
    L.grid = cfg_split(L.cfg) ? int64_t(s.dp_tiles) + s.tail_wgs : L.tiles;
  }
}

void fill_shampoo_descs(const ShampooPlan& sp, const shampoo_matrix* mats,
                        const shampoo_hparams* hp, char* ws, std::vector<MatDesc>* out) {
  const Plan& plan = sp.plan;
  out->assign(plan.mats.size(), MatDesc());
  auto slot_desc = [&](int e, int s) -> BufDesc {
    const PlanMat& p = plan.mats[size_t(e)];
    return {ws + p.off[s], p.mp, int32_t(p.m), int32_t(p.mp)};
  };
  for (int i = 0; i < sp.count; ++i) {
    const PlanMat& p = plan.mats[size_t(i)];
    const shampoo_matrix& x = mats[i];
    MatDesc& d = (*out)[size_t(i)];
    std::memset(&d, 0, sizeof d);
    char* g = ws + p.off[kShG];
    char* gt = ws + p.off[kShGT];
    char* z = ws + p.off[kShZ];
    d.grad = x.grad;
    d.mom = nullptr;
    d.copy_out = g;
    d.copy_ld = p.np;
    d.trans_out = gt;
    d.trans_ld = p.mp;
    d.rows = int32_t(p.r);
    d.cols = int32_t(p.c);
    const int64_t es = int64_t(p.esize);
    d.vec = ((uintptr_t)x.grad % 16 == 0 && (p.c * es) % 16 == 0) ? 1 : 0;
    d.wvec = ((uintptr_t)x.param % 16 == 0 && (p.c * es) % 16 == 0) ? 1 : 0;
    // bf16 W and G: the momentum kernel writes fp32 copies of G, and the fp32 kernel's update
    // rounds W to bf16.
    d.gram_f32 = p.dtype == kBF16 ? 1 : 0;
    d.buf[kShG] = {g, p.np, int32_t(p.r), int32_t(p.np)};
    d.buf[kShGT] = {gt, p.mp, int32_t(p.c), int32_t(p.mp)};
    d.buf[kShXL] = slot_desc(sp.left_entry[size_t(i)], sp.root_slot);
    d.buf[kShXR] = slot_desc(sp.right_entry[size_t(i)], sp.root_slot);
    d.buf[kShZ] = {z, p.np, int32_t(p.r), int32_t(p.np)};
    d.buf[kW] = {x.param, p.c, int32_t(p.r), 0};
    d.mom_prefix = int32_t(p.mom_prefix);
    d.mom_tiles_c = int32_t(p.mom_tiles_c);
    d.mom_tiles_r = int32_t(p.mom_tiles_r);
    d.full_prefix = int32_t(p.full_prefix);
    d.eta = hp->lr;
  }
  for (size_t j = 0; j < sp.stat_mat.size(); ++j) {
    const int e = sp.count + int(j);
    const PlanMat& p = plan.mats[size_t(e)];
    MatDesc& d = (*out)[size_t(e)];
    std::memset(&d, 0, sizeof d);
    for (int s = 0; s < sp.slots; ++s) d.buf[s] = slot_desc(e, s);
    // The factor F of S += F F^T: G for the left statistic (rows x cols), G^T for the right.
    d.buf[kShX] = sp.stat_right[j] ? (*out)[size_t(sp.stat_mat[j])].buf[kShGT]
                                   : (*out)[size_t(sp.stat_mat[j])].buf[kShG];
    // The momentum kernel reads the accumulated statistic (m x mp, zero padded) for its sum
    // of squares.
    d.grad = ws + p.off[sp.stat_slot];
    d.mom = nullptr;
    d.rows = int32_t(p.m);
    d.cols = int32_t(p.mp);
    d.vec = 1;
    d.wvec = 0;
    d.mom_prefix = int32_t(p.mom_prefix);
    d.mom_tiles_c = int32_t(p.mom_tiles_c);
    d.mom_tiles_r = int32_t(p.mom_tiles_r);
    d.tri_prefix = int32_t(p.tri_prefix);
    d.eta = 0.0f;
  }
}

std::string describe_shampoo_plan(const ShampooPlan& sp) {
  static const char* kKind[] = {"syrk", "poly", "prod", "xform", "update", "ident", "affine"};
  static const char* kLaunch[] = {"momentum", "norm", "gemm", "copy_in", "copy_out"};
  const Plan& plan = sp.plan;
  std::ostringstream os;
  os.precision(17);
  os << "{\"count\":" << sp.count << ",\"workspace\":" << plan.ws_bytes << ",\"levels\":" << plan.levels
     << ",\"flops\":" << plan.flops << ",\"bytes\":" << plan.bytes << ",\"iters\":" << sp.iters
     << ",\"slots\":" << sp.slots << ",\"stat_slot\":" << sp.stat_slot << ",\"root_slot\":" << sp.root_slot
     << ",\"desc_off\":" << plan.desc_off << ",\"scale_off\":" << plan.scale_off
     << ",\"partial_off\":" << plan.partial_off << ",\"mom_tiles\":" << plan.total_mom_tiles
     << ",\"units\":" << plan.units << ",\"split_cnt_off\":" << plan.split_cnt_off
     << ",\"split_cnt_n\":" << plan.split_cnt_n << ",\"split_slot_off\":" << plan.split_slot_off
     << ",\"split_slots\":" << plan.split_slots
     << ",\"entries\":[";
  for (size_t e = 0; e < plan.mats.size(); ++e) {
    const PlanMat& p = plan.mats[e];
    const bool stat = int(e) >= sp.count;
    os << (e ? "," : "") << "{\"kind\":\"" << (stat ? (sp.stat_right[e - size_t(sp.count)] ? "right" : "left") : "grad")
       << "\",\"dtype\":" << p.dtype << ",\"matrix\":" << p.orig << ",\"rows\":" << p.r << ",\"cols\":" << p.c << ",\"m\":" << p.m
       << ",\"tiles\":" << (stat ? p.tri_tiles : p.full_tiles) << ",\"mom_tiles\":" << p.mom_tiles
       << ",\"regions\":[";
    bool first = true;
    for (int b = 0; b < kNumBuf; ++b) {
      if (p.off[b] < 0) continue;
      const int64_t bytes = stat ? p.m * p.mp * 4 : (b == kShGT ? p.c * p.mp * 4 : p.r * p.np * 4);
      os << (first ? "" : ",") << "[" << p.off[b] << "," << bytes << "]";
      first = false;
    }
    os << "]}";
  }
  os << "],\"launches\":[";
  for (size_t i = 0; i < plan.launches.size(); ++i) {
    const PlanLaunch& L = plan.launches[i];
    os << (i ? "," : "") << "{\"kind\":\"" << kLaunch[L.kind] << "\",\"level\":" << L.level
       << ",\"first\":" << L.first << ",\"last\":" << L.last << ",\"tiles\":" << L.tiles
       << ",\"grid\":" << L.grid << ",\"cfg\":" << L.cfg << ",\"kmin\":" << L.kmin_cfg[0]
       << ",\"split\":{\"mode\":" << L.split_cfg[0].mode << ",\"c\":" << L.split_cfg[0].c
       << ",\"n\":" << L.split_cfg[0].n << ",\"dp_tiles\":" << L.split_cfg[0].dp_tiles
       << ",\"tail\":" << L.split_cfg[0].tail << ",\"tail_wgs\":" << L.split_cfg[0].tail_wgs
       << ",\"slots\":" << L.split_cfg[0].slots << "}"
       << ",\"buf_ok\":" << (L.buf_ok ? "true" : "false") << ",\"flops\":" << L.flops << ",\"coef\":[" << L.pa << "," << L.pb
       << "," << L.pc << "],\"groups\":[";
    for (size_t g = 0; g < L.groups.size(); ++g) {
      const GroupArg& a = L.groups[g];
      os << (g ? "," : "") << "{\"kind\":\"" << kKind[int(a.kind)] << "\",\"a\":" << int(a.a)
         << ",\"b\":" << int(a.b) << ",\"c\":" << int(a.c) << ",\"e\":" << int(a.e)
         << ",\"alpha\":" << int(a.alpha) << ",\"tri\":" << int(a.tri)
         << ",\"tile_begin\":" << a.tile_begin << "}";
    }
    os << "]}";
  }
  os << "]}";
  return os.str();
}

}  // namespace muon
