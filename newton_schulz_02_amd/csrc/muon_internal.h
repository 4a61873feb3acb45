// Internal types shared by the host planner and the gfx950 kernels of libmuon.
//
// Data layout in HBM (all row-major):
//   - caller buffers: W, G, M are rows x cols with leading dimension cols;
//   - per matrix, m = min(rows, cols), n = max(rows, cols), mp = round_up(m, 128),
//     np = round_up(n, 128);
//   - Gram slots (5 per matrix): m rows x mp columns, columns m..mp-1 held at zero so a
//     contraction may always run over mp;
//   - row form X (m x np) and transposed form X^T (n x mp), zero padded the same way.
//     When the caller's momentum buffer already has a 128-multiple leading dimension and
//     16-byte alignment it is used in place as one of the two forms.
#pragma once

#include <cstdint>

namespace muon {

constexpr int kTile = 256;       // output tile edge of the square-tile MFMA kernel
constexpr int kSmallTile = 128;  // output tile edge of the small-tile MFMA kernel
constexpr int kWideM = 256;      // output tile rows of the wide-tile MFMA kernel
constexpr int kWideN = 384;      // output tile columns of the wide-tile MFMA kernel
// MFMA kernel configurations (chosen per launch: tuned, or the square one by default):
// for 0..3, bit 0 is the tile shape (256 x 256 or 256 x 384) and bit 1 the tail split of the
// launch's last partial round of workgroups (tile_order.h); 4 is the 256 x 256 kernel with a
// deeper load pipeline (4 LDS stages of 64-byte rows, three k-steps of loads in flight); 5
// is the 128 x 128 kernel (4 waves of 64 x 64, two workgroups per compute unit), for
// launches with few tiles or short contractions.
enum GemmCfg : int32_t {
  kCfgSquare = 0,
  kCfgWide = 1,
  kCfgSquareSplit = 2,
  kCfgWideSplit = 3,
  kCfgSquareDeep = 4,
  kCfgSmall = 5,
  kNumCfg = 6
};
// Tile shapes: 256 x 256 (kCfgSquare), 256 x 384 (kCfgWide), 128 x 128 (kShapeSmall).
constexpr int kShapeSmall = 2;
constexpr int kNumShapes = 3;
inline int cfg_shape(int cfg) { return cfg == kCfgSmall ? kShapeSmall : (cfg & 1); }
inline bool cfg_split(int cfg) { return cfg == kCfgSquareSplit || cfg == kCfgWideSplit; }
inline bool cfg_deep(int cfg) { return cfg == kCfgSquareDeep; }
constexpr int kMaxUnits = 256;   // compute units a split plans for (MI355X: 256)
constexpr int kSplitUnit = 4;    // split pieces start and end on multiples of 4 k-steps
constexpr int64_t kSlotFloats = int64_t(kWideM) * kWideN;  // partial sums of one tile piece
constexpr int kKPad = 128;       // contraction dimensions are padded to this multiple
constexpr int kEwTile = 64;      // tile edge of the momentum/transpose kernel
constexpr int kMaxGroups = 8;    // op groups per grouped GEMM launch
constexpr int kSlots = 5;        // m x m Gram buffers per matrix
constexpr int64_t kStatusBytes = 256;  // head of every workspace: int32 status word (0 = ok)
constexpr size_t kNoAllocBytes = size_t(128) << 20;  // scratch of muon_step_noalloc, per device

enum DType : int32_t { kBF16 = 1, kF32 = 2 };

// Buffer ids inside MatDesc::buf.
enum BufId : int8_t {
  kSlot0 = 0,  // .. kSlot0 + kSlots - 1: Gram iterates G, P, Q, T
  kXrIn = 5,   // initial row form X (m x n)
  kXtIn = 6,   // initial transposed form X^T (n x m)
  kXrWs = 7,   // re-anchored row form
  kXtWs0 = 8,  // re-anchored transposed form, ping
  kXtWs1 = 9,  // re-anchored transposed form, pong
  kW = 10,     // the parameter (rows x cols), output of the update
  kNumBuf = 11
};

// Epilogue / op kinds of the grouped GEMM.
enum OpKind : int8_t {
  kOpSyrk = 0,    // C = alpha * A A^T, lower tiles, mirrored
  kOpPoly = 1,    // C = pa*I + pb*E + pc*(A B^T), lower tiles, mirrored
  kOpProd = 2,    // C = A B^T, lower tiles, mirrored
  kOpXform = 3,   // C = alpha * A B^T (full tiles) and C2 = its transpose
  kOpUpdate = 4,  // W -= eta * alpha * A B^T (full tiles)
  kOpIdent = 5,   // C = I (lower tiles, mirrored; no contraction)
  kOpAffine = 6   // C = alpha * (pa*I + pb*E) (lower tiles, mirrored; no contraction)
};

// alpha of an op: 1, the matrix's scale s, s^2, or s^(1/4).
enum AlphaMode : int8_t { kAlphaOne = 0, kAlphaS = 1, kAlphaS2 = 2, kAlphaQuarter = 3 };

struct BufDesc {
  void* ptr;
  int64_t ld;    // leading dimension in elements
  int32_t rows;  // valid rows
  int32_t kpad;  // columns to contract over when used as an operand (multiple of 64)
};

struct MatDesc {
  BufDesc buf[kNumBuf];
  const void* grad;      // caller G (rows x cols)
  void* mom;             // caller M (rows x cols), updated in place; null: M' = G, nothing stored
  void* copy_out;        // padded same-orientation copy of M' (rows x round_up(cols,kKPad)) or null
  void* trans_out;       // transposed copy of M' (cols x round_up(rows,kKPad)) or null
  int64_t copy_ld;
  int64_t trans_ld;
  int32_t rows, cols;
  int32_t vec;           // rows of G and M are 16-byte aligned: vector access allowed
  int32_t gram_f32;      // bf16 matrix iterating in fp32: its X copies and Gram slots are fp32,
                         // and the (fp32 kernel's) update rounds W to bf16
  int32_t wvec;          // rows of W are 16-byte aligned: vector access allowed
  int32_t mom_prefix;    // first momentum tile of this matrix (all matrices, sorted order)
  int32_t mom_tiles_c;   // momentum tiles along cols (cover round_up(cols, kKPad))
  int32_t mom_tiles_r;   // momentum tiles along rows (cover round_up(rows, kKPad))
  int32_t tri_prefix;    // first lower-triangle GEMM tile (prefix over sorted order)
  int32_t full_prefix;   // first full GEMM tile (prefix over sorted order)
  float eta;             // lr * sqrt(max(1, rows/cols))
  // The same prefixes for the wide-tile kernel: symmetric m x m outputs, full m x n
  // outputs, full n x m outputs (the update of a tall matrix).
  int32_t wide_prefix[3];
  // For the small-tile kernel: lower-triangle and full tiles.
  int32_t small_prefix[2];
};

struct GroupArg {
  int32_t first, last;   // matrix range [first, last) in the descriptor table
  int32_t tile_begin;    // first launch tile of this group
  int32_t tpm = 0;       // tiles per matrix when every matrix of the group has as many (the
                         // kernel then finds a tile's matrix by a division), else 0
  int8_t kind, a, b, c, c2, e, alpha, tri;  // c2 < 0: an xform stores no transposed copy
  int8_t nm;             // full output of n x m elements (the update of a tall matrix)
};

struct GemmArgs {
  const MatDesc* desc;
  const float* scale;    // per matrix s = 1 / (||M'||_F + eps)
  float pa, pb, pc;
  int32_t ngroups;
  int32_t total_tiles;   // output tiles of the launch
  int32_t grid;          // workgroups of the launch (total_tiles unless the tail is split)
  int32_t buf32;         // launcher only: every operand is below 2 GB, so the 256 x 256 kernel
                         // may address operands with 32-bit buffer offsets
  GroupArg g[kMaxGroups];
  // Tail split (tile_order.h): the first dp_tiles workgroups run whole tiles (all of them
  // when split_mode is kSplitNone), the next tail_wgs run pieces of the last tail_tiles.
  int32_t dp_tiles;
  int32_t split_mode, split_c, split_n;
  int32_t tail_tiles, tail_wgs;
  int32_t* split_cnt;    // 2 per tail tile: pieces done, partial sums written; 0 between launches
  float* split_slots;    // kSlotFloats per piece of a tail tile
  int32_t* status;       // the workspace's status word (split_protocol.h)
  int32_t split_spins;   // polls of a last piece's bounded wait (kSplitSpins)
};

struct MomArgs {
  const MatDesc* desc;
  float* partials;       // one partial sum of squares per momentum tile
  // The first launch of a step clears the workspace's status word and the tail-split
  // counters (workgroup 0, before any contraction of the step runs); null otherwise.
  int32_t* status;
  int32_t* split_cnt;
  int32_t split_cnt_n;
  int32_t first, last;   // matrix range [first, last) of one dtype
  int32_t tile_begin;    // mom_prefix of `first`
  int32_t total_tiles;   // tiles of the range
  float beta;
};

struct NormArgs {
  const MatDesc* desc;
  const float* partials;
  float* scale;
  int32_t count;
  float eps;
  int32_t* split_cnt;    // tail-split counters to clear before the contractions
  int32_t split_cnt_n;
};

struct AdamArgs {
  float* p;
  const float* g;
  float* m;
  float* v;
  int64_t n;
  float lr, beta1, beta2, eps, wd;
  float bc1, bc2;        // 1 - beta1^t, 1 - beta2^t (computed on the host in double)
};

inline int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }
inline int64_t ceil_div(int64_t x, int64_t q) { return (x + q - 1) / q; }

}  // namespace muon

// Kernel launchers (defined in the .hip files).  Each returns a hipError_t as int.
int muon_launch_momentum(const muon::MomArgs& a, int dtype, void* stream);
int muon_launch_norm(const muon::NormArgs& a, void* stream);
int muon_launch_gemm(const muon::GemmArgs& a, int dtype, void* stream);
int muon_launch_gemm_deep(const muon::GemmArgs& a, int dtype, void* stream);
int muon_launch_gemm_small(const muon::GemmArgs& a, int dtype, void* stream);
int muon_launch_gemm_wide(const muon::GemmArgs& a, int dtype, void* stream);
int muon_launch_adamw(const muon::AdamArgs& a, void* stream);
// noalloc.hip: device address of the allocation-free entry point's scratch array on device
// `dev` (asked of the runtime once per device; that device must be current), and a copy of
// a small host block (bytes a multiple of 4) to device memory through kernel arguments.
int muon_noalloc_scratch(int dev, void** ptr);
int muon_put_words(void* dst, const void* src, size_t bytes, void* stream);
