// Host-side planning of one shampoo_step call (include/shampoo.h): validation, the op
// schedule of the statistics and their inverse fourth roots, slot assignment, workspace
// layout and the grouped launch list.  Pure C++: no HIP call.
//
// The plan reuses the Muon launch machinery: its "matrices" are descriptor entries of two
// kinds.  Entries [0, count) are the caller's matrices (gradient entries: the copies of G,
// the product X_L G and the update of W); entries [count, 3 count) are the statistics, the
// left one (rows x rows) and the right one (cols x cols) of every matrix, in decreasing size
// (statistic entries: the accumulation and the coupled Newton iteration).  Every statistic
// runs the same schedule, so each dependency level is one grouped launch over all of them.
#pragma once

#include <string>
#include <vector>

#include "../../include/shampoo.h"
#include "planner.h"

namespace muon {

// Buffer ids (MatDesc::buf) of the two kinds of entries.
enum ShampooBuf : int8_t {
  // gradient entries (and kW for the parameter)
  kShG = 0,   // G, rows x round_up(cols, kKPad), zero padded
  kShGT = 1,  // G^T, cols x round_up(rows, kKPad), zero padded
  kShXL = 2,  // the left root X_L: the finished slot of the left statistic entry
  kShXR = 3,  // the right root X_R: the finished slot of the right statistic entry
  kShZ = 4,   // X_L G, rows x round_up(cols, kKPad)
  // statistic entries: slots 0 .. kShSlots - 1 (m x round_up(m, kKPad) fp32), and
  kShX = 8    // the factor of the accumulation: G (left statistic) or G^T (right), m rows
};
constexpr int kShSlots = 7;
constexpr int64_t kShMaxDim = 65536;
constexpr int kShMaxIters = 64;

struct ShampooPlan {
  Plan plan;                        // entries (plan.mats), launches and workspace offsets
  int count = 0;                    // caller matrices
  std::vector<int> stat_mat;        // statistic entry count + j -> caller matrix
  std::vector<int8_t> stat_right;   // statistic entry count + j: 1 for the right statistic
  std::vector<int> left_entry, right_entry;  // caller matrix -> its statistic entries
  int stat_slot = 0;                // slot that holds the accumulated statistic
  int root_slot = 0;                // slot that holds the finished root
  int slots = 0;                    // slots per statistic entry
  int iters = 0;
};

// Validate and plan.  Returns MUON_OK or a negative muon_status with *err set.
int build_shampoo_plan(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                       ShampooPlan* sp, std::string* err);

// Tail splits of the MFMA launches for `units` compute units (capped at kMaxUnits).
// force_cfg < 0: split every launch that has a tail worth cutting (except the accumulation,
// which runs before the split counters are cleared); otherwise split only when
// cfg_split(force_cfg).  build_shampoo_plan calls it with kMaxUnits and -1.
void shampoo_plan_splits(ShampooPlan* sp, int units, int force_cfg);

// Fill the device descriptor table for a concrete workspace base address.
void fill_shampoo_descs(const ShampooPlan& sp, const shampoo_matrix* mats,
                        const shampoo_hparams* hp, char* ws, std::vector<MatDesc>* out);

std::string describe_shampoo_plan(const ShampooPlan& sp);

}  // namespace muon
