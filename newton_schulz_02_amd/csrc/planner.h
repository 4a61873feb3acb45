// Host-side planning of one muon_step call: validation, shape buckets, restart sets,
// the per-matrix op schedule in Gram space, Gram-slot assignment, workspace layout and
// the grouped launch list.  Pure C++: no HIP call, so it runs (and is tested) without a GPU.
#pragma once

#include <functional>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "muon_internal.h"
#include "tile_order.h"

namespace muon {

struct PlanOp {
  int8_t kind, a, b, c, c2, e, alpha, tri;
  int level;
  bool same_sig(const PlanOp& o) const {
    return kind == o.kind && a == o.a && b == o.b && c == o.c && c2 == o.c2 && e == o.e &&
           alpha == o.alpha && tri == o.tri;
  }
};

struct PlanMat {
  int orig = 0;                  // index in the caller's list
  int64_t r = 0, c = 0, m = 0, n = 0, mp = 0, np = 0;
  bool tall = false;
  int dtype = kBF16;              // the caller's buffers (G, M, W)
  size_t esize = 2;
  int gdtype = kBF16;             // the Gram iterates, X forms and contractions (gram_dtype)
  size_t gsize = 2;
  uint32_t restarts = 0;
  std::vector<PlanOp> ops;
  int64_t off[kNumBuf];          // workspace offsets of workspace-resident buffers, -1 if none
  int64_t copy_off = -1;         // reserved padded same-orientation copy
  int64_t trans_off = -1;        // reserved transposed copy
  int64_t tri_tiles = 0, full_tiles = 0, mom_tiles = 0, mom_tiles_c = 0, mom_tiles_r = 0;
  int64_t tri_prefix = 0, full_prefix = 0, mom_prefix = 0;
  // Wide-tile kernel: tiles of a symmetric m x m, a full m x n and a full n x m output, and
  // their prefixes over the sorted order.
  int64_t wide_tiles[3] = {0, 0, 0}, wide_prefix[3] = {0, 0, 0};
  // Small-tile kernel: tiles of a symmetric m x m and of a full m x n output, and prefixes.
  int64_t small_tiles[2] = {0, 0}, small_prefix[2] = {0, 0};
  bool wide_ok = true;  // every operand fits the 256 x 384 kernel's 32-bit buffer offsets
  bool buf_ok = true;   // every operand (rows x leading dimension) is below 2 GB
  double flops = 0, bytes = 0;
};

// kLaunchCopyIn / kLaunchCopyOut (Shampoo): copy the caller's statistics of entries
// [first, last) into their workspace slot, and back.
enum LaunchKind {
  kLaunchMomentum = 0,
  kLaunchNorm = 1,
  kLaunchGemm = 2,
  kLaunchCopyIn = 3,
  kLaunchCopyOut = 4
};

struct PlanLaunch {
  int kind = kLaunchGemm;
  int dtype = kBF16;
  int level = -1;
  int first = 0, last = 0;       // momentum: matrix range
  std::vector<GroupArg> groups;  // gemm: the groups of the chosen kernel configuration
  int64_t tiles = 0;
  int cfg = kCfgSquare;          // gemm: the chosen MFMA kernel configuration (GemmCfg)
  int64_t grid = 0;              // gemm: workgroups of the chosen configuration
  std::vector<GroupArg> groups_cfg[kNumShapes];  // gemm: the groups under each tile shape
  int64_t tiles_cfg[kNumShapes] = {0, 0, 0};
  int kmin_cfg[kNumShapes] = {0, 0, 0};  // gemm: fewest k-steps among the last kMaxUnits tiles
  SplitPlan split_cfg[kNumShapes];     // gemm: tail split under each tile shape
  bool wide_ok = true;           // gemm: the 256 x 384 configuration may run this launch
  bool buf_ok = true;            // gemm: every operand is below 2 GB (32-bit buffer offsets)
  bool own_coef = false;         // gemm: pa, pb, pc below (else the Newton-Schulz a, b, c)
  float pa = 0.0f, pb = 0.0f, pc = 0.0f;
  std::string signature;         // gemm: shapes and ops of the launch (the tuning key)
  double flops = 0, bytes = 0;
};

struct Plan {
  std::vector<PlanMat> mats;     // sorted order
  std::vector<PlanLaunch> launches;
  int64_t desc_off = 0, scale_off = 0, partial_off = 0;
  // Tail split: 2 counters per tail tile and one partial-sum slot per piece.
  int64_t split_cnt_off = 0, split_slot_off = 0;
  int32_t split_cnt_n = 0;
  int64_t split_slots = 0;
  int units = kMaxUnits;         // compute units the splits are planned for
  int64_t total_mom_tiles = 0;
  size_t ws_bytes = 0;
  int levels = 0;
  double flops = 0, bytes = 0;
};

// Chooses the MFMA kernel configuration of a launch from its signature, or -1 for the default
// (default_cfg).
using CfgChooser = std::function<int(const std::string& signature)>;

// Configuration of a launch that no table entry or force names: the 128 x 128 tiles for a
// launch of fewer than kSmallDefaultTiles tiles of 256 x 256 (measured: a lone 256 x 1024
// fp32 matrix, 1 to 16 such tiles per launch, runs 2.4 times faster on them; 160 tiles per
// launch tie, 952 or more run 15 % slower), else the 256 x 256 tiles.
constexpr int64_t kSmallDefaultTiles = 64;
inline int default_cfg(int64_t square_tiles) {
  return square_tiles < kSmallDefaultTiles ? kCfgSmall : kCfgSquare;
}

// Validate and plan.  Returns MUON_OK or a negative muon_status with *err set.  Without a
// chooser every launch uses its default configuration (default_cfg).
int build_plan(const muon_matrix* mats, int32_t count, const muon_hparams* hp, Plan* plan,
               std::string* err, const CfgChooser* choose = nullptr);

// Plan the tail split of every MFMA launch for `units` compute units (capped at
// kMaxUnits) and apply the chosen configurations' grids.  build_plan calls it with
// kMaxUnits; a device with fewer units re-plans before launching.
void plan_splits(Plan* plan, int units);

// Fill the device descriptor table for a concrete workspace base address.
void fill_descs(const Plan& plan, const muon_matrix* mats, const muon_hparams* hp, char* ws,
                std::vector<MatDesc>* out);

// Dtype of a matrix's Gram iteration: bf16 matrices with m <= kF32GramMaxM iterate in fp32.
// With few Gram rows each bf16 product sums few terms, so the rounding of the stored iterates
// does not average out; measured on thin bf16 matrices (m <= 48, n up to 8192) it took the
// result past the 2e-2 bar (up to 7e-2 at m = 4), while m >= 64 stayed near 1e-2.  The fp32
// products of such small Gram spaces cost little next to the bf16 contractions over n.  Their
// Gram formation and update then run in the fp32 kernel on fp32 copies of X, and the update
// rounds W back to bf16.
constexpr int64_t kF32GramMaxM = 128;

// fp32 launches whose tail tiles contract over at least this many elements run with the tail
// split whatever the chosen configuration: the MFMA accumulates a tile's products in fp32 in
// sequence, so its rounding error grows as the square root of the contraction length; at
// 2^20 (the longest side allowed) that took a 3 x 2^20 fp32 matrix to 1.3e-4 relative error
// against the 1e-4 bar.  Split pieces keep separate fp32 sums, added in piece order: eighths
// of the contraction when a launch has at most units/8 tail tiles, units/R-ths for R up to
// units/2, halves or so beyond that (tile_order.h, plan_split).  A launch of fewer tiles than
// units is all tail; the whole-round tiles of a bigger one are not cut.
constexpr int64_t kF32SplitMinK = int64_t(1) << 17;
int gram_dtype(int dtype, int64_t m);

// Resolve the restart set of one matrix (bit k = re-anchor before iteration k).
uint32_t resolve_restarts(uint32_t mask, int64_t m, int64_t n, int steps);

std::string describe_plan(const Plan& plan);

}  // namespace muon
