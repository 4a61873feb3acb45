// Wide-tile variant of the grouped MFMA contraction kernel of the Gram Newton-Schulz step,
// for gfx950 (CDNA4).  It computes the same ops on the same operands as the square-tile
// kernel (kernels_gemm.hip): C = A B^T with both operands row-major and the contraction
// index contiguous, several op groups per launch (DMuon summary §2.2, batching of similar
// shapes), symmetric outputs on the tiles holding elements on or below the diagonal with
// mirror-on-store (DMuon summary §2.2, SYRK-type path).  Its output tile is kWideM x kWideN
// (256 x 384) instead of 256 x 256; the step picks one of the two kernels per launch.
//
// Why a wider tile.  The main loop of these kernels is bound by the L1-to-L2 requests of the
// operand loads (one per 128-byte line; a CU keeps a limited number in flight), not by MFMA
// issue.  A 256 x 384 tile needs 640 requests per k-step for 1.5 times the work of a
// 256 x 256 tile (512 requests), and it splits a level into fewer, larger rounds of
// workgroups.  Its 192 fp32 accumulators per lane (8 waves) leave 64 registers for
// everything else, which shapes the code below:
//   * operands are loaded with buffer instructions straight to LDS
//     (buffer_load_dwordx4 ... lds): the per-lane part of an address is one 32-bit offset
//     (row and chunk), the k-step's part the scalar offset; rows past the end of an operand
//     (offsets at or beyond rows x row pitch) read as zeros, so no per-lane clamp is kept;
//   * one scheduling barrier per MFMA block keeps the fragment reads of the next block
//     from being hoisted (and held in registers) early;
//   * the epilogue is per wave: each wave stores its 128 x 96 block one 32-row slab at a
//     time through a private LDS slab, so the accumulators free up slab by slab and no
//     workgroup barrier is needed.
//
// Main loop: 8 waves in a 2 x 4 grid, each owning 128 x 96 = 4 x 3 blocks of 32 x 32 MFMA
// accumulators (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x2_f32 for fp32).  A stage
// holds 128 bytes of every operand row: 256 A rows (32 KB) and 384 B rows (48 KB); the two
// stages fill the CU's 160 KB of LDS.  The 16-byte chunk c of LDS row r sits at chunk
// position c ^ ((r / 2) mod 8), so the 16 rows of a fragment read hit 16 distinct bank
// groups.  Each stage is its own __shared__ array and the k loop is unrolled by two, so
// every LDS access names its array statically and the fragment reads do not wait for the
// loads in flight to the other stage.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "muon_internal.h"
#include "split_fixup.h"
#include "tile_order.h"

using namespace muon;


namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWavesM = 2;                      // waves along the tile rows
constexpr int kWavesN = 4;                      // waves along the tile columns
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveRows = kWideM / kWavesM;     // 128
constexpr int kWaveCols = kWideN / kWavesN;     // 96
constexpr int kFragM = kWaveRows / 32;          // 32-row blocks per wave (4)
constexpr int kFragN = kWaveCols / 32;          // 32-column blocks per wave (3)
constexpr int kStages = 2;
constexpr int kRowBytes = 128;                  // bytes of one operand row per stage
constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row
constexpr int kABytes = kWideM * kRowBytes;     // A rows of a stage (32 KB)
constexpr int kBBytes = kWideN * kRowBytes;     // B rows of a stage (48 KB)
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kRowsPerInst = 1024 / kRowBytes;  // rows one wave instruction fills
constexpr int kInstA = kABytes / 1024 / kWaves; // load instructions per wave per stage
constexpr int kInstB = kBBytes / 1024 / kWaves;
constexpr int kLoadsPerStage = kInstA + kInstB;
constexpr int kArrBytes = kStageBytes;
static_assert(kStages * kArrBytes <= 160 * 1024, "LDS budget");
static_assert(kInstA >= 1 && kInstB >= 1 && kInstA * kWaves * 1024 == kABytes &&
              kInstB * kWaves * 1024 == kBBytes, "every wave loads part of each operand");
static_assert(kKPad % (kStages * kRowBytes / 4) == 0 && kKPad % (kStages * kRowBytes / 2) == 0,
              "padded contraction dims must hold whole blocks of stages");
static_assert(kFragM == 4, "four 32-row slabs per wave");

// Chunk position of 16-byte chunk c in LDS row r is c ^ swz(r) (a bijection on a row).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float to_f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ float to_f(float f) { return f; }
__device__ __forceinline__ uint16_t from_f(float f, uint16_t*) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float from_f(float f, float*) { return f; }

// MFMA step over one 16-byte fragment per operand.
template <typename S>
struct Mma;

template <>
struct Mma<uint16_t> {
  static constexpr int kStageK = kRowBytes / 2;   // k elements per stage
  __device__ __forceinline__ static void step(const uint4& a, const uint4& b, f32x16& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int kStageK = kRowBytes / 4;
  // The fragment holds 4 consecutive k values per lane; MFMA e contracts over element e
  // of both operands (A and B use the same k map, so the sum covers all 8 k values).
  __device__ __forceinline__ static void step(const uint4& a, const uint4& b, f32x16& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14].
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Workgroup barrier for the main loop.  __syncthreads() carries a release fence that
// would wait for every load in flight (LDS-DMA loads count as LDS writes), draining the
// pipeline; here each wave has already waited for the loads of the stage it is about to
// read (wait_vm), and its LDS reads of the previous stage completed before the MFMAs that
// consumed them.  The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Calls f(integral_constant<int, S>) for S = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Global-memory pointers.  Pointers read from the descriptor table are generic; accesses
// through them would compile to FLAT instructions, which may alias LDS, so every wait for
// an LDS access would also wait for them.  The epilogue casts to address space 1 instead.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> to_global(T* p) {
  return (gptr<T>)(p);
}

// Eight consecutive elements of S as one 16- or 32-byte vector.
template <typename S>
struct Vec8 {
  S v[8];
};
template <typename S>
__device__ __forceinline__ void load8(gptr<const S> p, Vec8<S>& x) {
  const gptr<const u32x4> q = (gptr<const u32x4>)p;
  reinterpret_cast<u32x4*>(x.v)[0] = q[0];
  if constexpr (sizeof(S) == 4) reinterpret_cast<u32x4*>(x.v)[1] = q[1];
}
template <typename S>
__device__ __forceinline__ void store8(gptr<S> p, const Vec8<S>& x) {
  const gptr<u32x4> q = (gptr<u32x4>)p;
  q[0] = reinterpret_cast<const u32x4*>(x.v)[0];
  if constexpr (sizeof(S) == 4) q[1] = reinterpret_cast<const u32x4*>(x.v)[1];
}

// Value of the symmetric-output epilogues at (gi, gj); x is the accumulated product.  E is
// read at (er, ec), which is (gi, gj) or its mirror: stored iterates are exactly symmetric.
template <typename S>
__device__ __forceinline__ float tri_value(int kind, int gi, int gj, int m, float x, float alpha,
                                           gptr<const S> E, int64_t lde, int er, int ec, float pa,
                                           float pb, float pc) {
  if (gi >= m || gj >= m) return 0.0f;
  if (kind == kOpSyrk) return alpha * x;
  if (kind == kOpPoly) return (gi == gj ? pa : 0.0f) + pb * to_f(E[int64_t(er) * lde + ec]) + pc * x;
  if (kind == kOpIdent) return gi == gj ? 1.0f : 0.0f;
  return x;
}

// ---- per-wave epilogue ---------------------------------------------------------------
// A wave's 128 x 96 block is stored one 32-row slab at a time.  The slab's values are formed
// in registers and written transposed into the wave's private LDS slab: T-row c (a column of
// the block) holds the slab's 32 values, in the staging type (bf16 bits for bf16 outputs of
// the Gram ops, fp32 for the update and for fp32 outputs).  Two copy passes follow:
// transposed (row c of C^T gets 32 consecutive values) and direct (8 consecutive columns of
// one row, gathered from 8 T-rows; 32 consecutive lanes take 32 consecutive rows).
constexpr int kSlabRows = 32;
template <typename T>
constexpr int slab_ld() { return kSlabRows + 16 / int(sizeof(T)); }  // 16-byte pad per T-row
constexpr int kSlabBytes = kWaveCols * (kSlabRows + 4) * 4;          // fp32 staging, the larger
static_assert(kWaves / 2 * kSlabBytes + 16 <= kArrBytes,
              "per-wave slabs fit the stage arrays, clear of the split flags at the end of lds0");

template <typename S>
struct EpArgs {
  float alpha, pa, pb, pc, step;
  gptr<S> C, T;
  gptr<const S> E;
  int64_t ldc, ldt, lde;
  int rows_out, cols_out, m, d_rows, d_cols, t_rows, t_cols, wvec;
  int wbf16;    // the update's W is bf16 (a bf16 matrix whose Gram iteration ran in fp32)
  int r0, c0;   // first row and column of the wave's block
  int lane;
};

template <int K, typename S>
__device__ __attribute__((always_inline)) inline void ep_wave(f32x16 (&acc)[kFragM][kFragN],
                                                             const EpArgs<S>& e, char* slab_bytes) {
  // Staging type: fp32 for the update and for fp32 outputs, else the bf16 bits.
  using T = std::conditional_t<(K == kOpUpdate || sizeof(S) == 4), float, uint16_t>;
  constexpr int ld = slab_ld<T>();
  T* slab = reinterpret_cast<T*>(slab_bytes);
  const int lr = e.lane & 31, lk = e.lane >> 5;
  const bool sym = !(K == kOpXform || K == kOpUpdate);
#pragma unroll
  for (int i = 0; i < kFragM; ++i) {
    const int sr0 = e.r0 + 32 * i;  // first row of the slab
    // 1. Values of the slab, written transposed.
    u32x2 e4[kFragN][4];
    if constexpr (K == kOpPoly) {
#pragma unroll
      for (int j = 0; j < kFragN; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int gi0 = sr0 + 8 * r4 + 4 * lk, gj = e.c0 + 32 * j + lr;
          e4[j][r4] = u32x2{0u, 0u};
          if (gj < e.m && gi0 < e.m) e4[j][r4] = *(gptr<const u32x2>)(e.E + int64_t(gj) * e.lde + gi0);
        }
    }
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int lrow = 8 * r4 + 4 * lk, lcol = 32 * j + lr;
        const int gi0 = sr0 + lrow, gj = e.c0 + lcol;
        T o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gi = gi0 + q;
          const float x = acc[i][j][4 * r4 + q];
          float val;
          if constexpr (K == kOpUpdate) {
            val = x;
          } else if constexpr (K == kOpXform) {
            val = (gi < e.rows_out && gj < e.cols_out) ? e.alpha * x : 0.0f;
          } else {
            const bool in = gi < e.m && gj < e.m;
            if constexpr (K == kOpSyrk) val = in ? e.alpha * x : 0.0f;
            else if constexpr (K == kOpPoly) {
              float ev;
              if constexpr (sizeof(S) == 2) ev = to_f(reinterpret_cast<const uint16_t*>(&e4[j][r4])[q]);
              else ev = e.E[int64_t(gj) * e.lde + gi];
              val = in ? (gi == gj ? e.pa : 0.0f) + e.pb * ev + e.pc * x : 0.0f;
            } else if constexpr (K == kOpIdent) val = (in && gi == gj) ? 1.0f : 0.0f;
            else val = in ? x : 0.0f;
          }
          if constexpr (sizeof(T) == 2) o[q] = from_f(val, static_cast<uint16_t*>(nullptr));
          else o[q] = val;
        }
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint2*>(slab + lcol * ld + lrow) = *reinterpret_cast<const uint2*>(o);
        else
          *reinterpret_cast<float4*>(slab + lcol * ld + lrow) = *reinterpret_cast<const float4*>(o);
      }
    // 2. Transposed pass: row gj of the transposed output gets the slab's 32 values of
    //    column gj, 8 at a time (the update has none).
    if constexpr (K != kOpUpdate) {
      for (int idx = e.lane; idx < kWaveCols * (kSlabRows / 8); idx += 64) {
        const int c = idx / (kSlabRows / 8), q8 = (idx % (kSlabRows / 8)) * 8;
        const int gj = e.c0 + c, gi = sr0 + q8;
        if (gj >= e.t_rows || gi >= e.t_cols) continue;
        if (sym && gi + 7 <= gj) continue;  // chunk on or above the diagonal
        Vec8<S> v;
#pragma unroll
        for (int q = 0; q < 8; ++q) v.v[q] = S(slab[c * ld + q8 + q]);
        if (!sym || (gi > gj && gi + 7 < e.t_cols)) {
          store8(e.T + int64_t(gj) * e.ldt + gi, v);
        } else {
          for (int q = 0; q < 8; ++q)
            if (gi + q > gj && gi + q < e.t_cols) e.T[int64_t(gj) * e.ldt + gi + q] = v.v[q];
        }
      }
    }
    // 3. Direct pass: row gi gets columns gj .. gj+7 of the slab.
    for (int idx = e.lane; idx < kSlabRows * (kWaveCols / 8); idx += 64) {
      const int r = idx % kSlabRows, c8 = (idx / kSlabRows) * 8;
      const int gi = sr0 + r, gj = e.c0 + c8;
      if constexpr (K == kOpUpdate) {  // W -= eta * alpha * (A B^T)
        if (gi >= e.rows_out || gj >= e.cols_out) continue;
        // W's element type Wt: S, or bf16 for a bf16 matrix whose Gram iteration ran in fp32.
        auto update = [&](auto wt) {
          using Wt = decltype(wt);
          const gptr<Wt> pw = (gptr<Wt>)(e.C) + int64_t(gi) * e.ldc + gj;
          if (e.wvec && gj + 7 < e.cols_out) {
            Vec8<Wt> w;
            load8<Wt>(pw, w);
#pragma unroll
            for (int q = 0; q < 8; ++q)
              w.v[q] = from_f(fmaf(-e.step, slab[(c8 + q) * ld + r], to_f(w.v[q])), static_cast<Wt*>(nullptr));
            store8(pw, w);
          } else {
            for (int q = 0; q < 8 && gj + q < e.cols_out; ++q)
              pw[q] = from_f(fmaf(-e.step, slab[(c8 + q) * ld + r], to_f(pw[q])), static_cast<Wt*>(nullptr));
          }
        };
        if (sizeof(S) == 4 && e.wbf16) update(uint16_t());
        else update(S());
      } else {
        if (gi >= e.d_rows || gj >= e.d_cols) continue;
        if (sym && gi < gj) continue;  // chunk above the diagonal
        Vec8<S> v;
#pragma unroll
        for (int q = 0; q < 8; ++q) v.v[q] = S(slab[(c8 + q) * ld + r]);
        if (!sym || (gi >= gj + 7 && gj + 7 < e.d_cols)) {
          store8(e.C + int64_t(gi) * e.ldc + gj, v);
        } else {
          for (int q = 0; q < 8; ++q)
            if (gi >= gj + q && gj + q < e.d_cols) e.C[int64_t(gi) * e.ldc + gj + q] = v.v[q];
        }
      }
    }
  }
}

// One output tile of the launch (logical tile `bid`), or piece `piece` of `pieces` of it when
// the tail split cut its contraction (cnt: the tile's two split counters, slots: its
// `pieces` partial-sum slots).
template <typename S>
__device__ __forceinline__ void gemm_wide_tile(const GemmArgs& args, const int bid, const int piece,
                                               const int pieces, int32_t* const cnt,
                                               float* const slots) {
  __shared__ __attribute__((aligned(1024))) char lds0[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kArrBytes];
  // The tail split's flags (split_fixup): the last 16 bytes of lds0, which the epilogue's
  // slabs leave alone (the two stages fill the LDS, so they get no array of their own).
  int* const split_flags = reinterpret_cast<int*>(lds0 + kArrBytes - 16);
  // Stage array s, named statically when s is a compile-time constant.
  auto stage_of = [&](auto sc) __attribute__((always_inline)) -> char* {
    if constexpr (decltype(sc)::value % kStages == 0) return lds0;
    else return lds1;
  };

  // ---- which group, matrix and tile --------------------------------------------------
  GroupArg g = args.g[0];
#pragma unroll
  for (int q = 1; q < kMaxGroups; ++q)
    if (q < args.ngroups && args.g[q].tile_begin <= bid) g = args.g[q];
  const MatDesc* desc = args.desc;
  // Tile prefixes of this group's output shape: symmetric, full m x n or full n x m.
  // The tile's matrix: a division when the group's matrices have equal tile counts, else a
  // binary search over the prefixes.
  const int sel = g.tri ? 0 : (g.nm ? 2 : 1);
  int lo, t;
  if (g.tpm > 0) {
    const int u = bid - g.tile_begin;
    lo = g.first + u / g.tpm;
    t = u % g.tpm;
  } else {
    const int v = bid - g.tile_begin + desc[g.first].wide_prefix[sel];
    int hi = g.last - 1;
    lo = g.first;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int pre = desc[mid].wide_prefix[sel];
      if (pre <= v) lo = mid; else hi = mid - 1;
    }
    t = v - desc[lo].wide_prefix[sel];
  }
  const MatDesc& d = desc[lo];

  const BufDesc C = d.buf[g.c];
  const int kind = g.kind;
  const bool ident = kind == kOpIdent;
  const BufDesc A = ident ? C : d.buf[g.a];
  const BufDesc B = ident ? C : d.buf[g.b];
  const int rows_out = A.rows;
  const int cols_out = B.rows;
  int ti, tj;
  if (g.tri) {
    sym_decode(t, rows_out, kWideM, kWideN, ti, tj);
  } else {
    full_band_decode(t, ceil_div_i(rows_out, kWideM), ceil_div_i(cols_out, kWideN), ti, tj);
  }
  const int row0 = ti * kWideM;
  const int col0 = tj * kWideN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN;   // 0..1: rows [128 wm, 128 wm + 128)
  const int wn = wave % kWavesN;   // 0..3: cols [96 wn, 96 wn + 96)
  const int lr = lane & 31;
  const int lk = lane >> 5;
  // In a tile crossing the diagonal of a symmetric output, a wave whose block lies strictly
  // above the diagonal computes nothing that is stored.
  const bool above = g.tri && row0 + kWaveRows * wm + kWaveRows - 1 < col0 + kWaveCols * wn;
  const bool idle = above || ident;

  f32x16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- loads: wave `wave` fills rows [wave*RA, wave*RA + RA) of A and [wave*RB, ...) of B
  // per stage, RA = kInstA * kRowsPerInst, RB = kInstB * kRowsPerInst, one instruction per
  // kRowsPerInst rows.  Lane l of an instruction writes LDS bytes [16 l, 16 l + 16) of its
  // 1 KB block: row l / kChunks of the block, chunk position l % kChunks, holding global
  // chunk (position ^ swz(row)).  Loads go through buffer resources: the per-lane byte
  // offset (row and chunk) is a 32-bit VGPR, the k-step's offset the scalar offset, and rows
  // past the end of an operand (offsets at or beyond its row count times its row pitch) read
  // as zeros.
  const int ksteps = ident ? 0 : A.kpad / Mma<S>::kStageK;
  int k0 = 0, k1 = ksteps;  // the k-steps of this piece
  if (pieces > 1) split_range(args.split_mode, args.split_n, ksteps, kSplitUnit, piece, pieces, k0, k1);
  const uint32_t lda = uint32_t(A.ld) * uint32_t(sizeof(S));
  const uint32_t ldb = uint32_t(B.ld) * uint32_t(sizeof(S));
  const int lrow = lane / kChunks;
  const int lpos = lane % kChunks;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(A.ptr), (short)0, int(uint32_t(A.rows) * lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(B.ptr), (short)0, int(uint32_t(B.rows) * ldb), 0x00020000);
  uint32_t a_off[kInstA], b_off[kInstB];
#pragma unroll
  for (int j = 0; j < kInstA; ++j) {
    const int r = (wave * kInstA + j) * kRowsPerInst + lrow;  // tile row
    a_off[j] = uint32_t(row0 + r) * lda + uint32_t((lpos ^ swz(r)) * 16);
  }
#pragma unroll
  for (int j = 0; j < kInstB; ++j) {
    const int r = (wave * kInstB + j) * kRowsPerInst + lrow;
    b_off[j] = uint32_t(col0 + r) * ldb + uint32_t((lpos ^ swz(r)) * 16);
  }
  // Issue the loads of k-step ks into stage array st.
  auto issue = [&](int ks, char* st) __attribute__((always_inline)) {
    const int koff = ks * kRowBytes;
#pragma unroll
    for (int j = 0; j < kInstA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void*)(st + (wave * kInstA + j) * 1024), 16,
                                               a_off[j], koff, 0, 0);
#pragma unroll
    for (int j = 0; j < kInstB; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_void*)(st + kABytes + (wave * kInstB + j) * 1024),
                                               16, b_off[j], koff, 0, 0);
  };
  // Prologue: stages 0 .. kStages-2 in flight.
  static_for<0, kStages - 1>([&](auto sc) {
    if (k0 + sc.value < k1) issue(k0 + sc.value, stage_of(sc));
  });

  // Fragment rows of this lane (+ 32 i for A, + 32 j for B).
  const int a_row = wm * kWaveRows + lr;
  const int b_row = wn * kWaveCols + lr;
  constexpr int kKK = kRowBytes / 32;  // MFMA k-blocks per step
  // Fragments of k-block kk (16-byte chunk 2 kk + lk of the lane's rows) from stage st.
  auto load_frags = [&](const char* st, int kk, uint4* fa, uint4* fb) __attribute__((always_inline)) {
    const int c = 2 * kk + lk;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
      const int r = a_row + 32 * i;
      fa[i] = *reinterpret_cast<const uint4*>(st + r * kRowBytes + ((c ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < kFragN; ++j) {
      const int r = b_row + 32 * j;
      fb[j] = *reinterpret_cast<const uint4*>(st + kABytes + r * kRowBytes + ((c ^ swz(r)) << 4));
    }
  };
  // One k-step: wait until this wave's loads of stage ks landed (at most `pending` newer
  // loads remain), barrier, issue the loads kStages-1 steps ahead, run the MFMAs.
  auto kstep = [&](int ks, auto sc, auto pending) __attribute__((always_inline)) {
    wait_vm<decltype(pending)::value>();
    stage_barrier();  // all waves' loads of stage ks landed; stage ks-1 is free again
    if (ks + kStages - 1 < k1)
      issue(ks + kStages - 1, stage_of(std::integral_constant<int, decltype(sc)::value + kStages - 1>{}));
    if (idle) return;
    const char* st = stage_of(sc);
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      uint4 fa[kFragM], fb[kFragN];
      load_frags(st, kk, fa, fb);
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) Mma<S>::step(fa[i], fb[j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // k0 and k1 are multiples of kStages (contraction dims are padded to kKPad, split pieces
  // end on multiples of kSplitUnit).  Full blocks keep kStages-2 stages in flight behind the
  // one being read; the last block drains.
  int kb = k0;
  for (; kb + kStages < k1; kb += kStages) {
    static_for<0, kStages>([&](auto sc) {
      kstep(kb + sc.value, sc, std::integral_constant<int, (kStages - 2) * kLoadsPerStage>{});
    });
  }
  if (kb < k1) {
    static_for<0, kStages>([&](auto sc) {
      constexpr int left = kStages - 1 - decltype(sc)::value;   // stages after this one
      constexpr int ahead = left < kStages - 2 ? left : kStages - 2;
      kstep(kb + sc.value, sc, std::integral_constant<int, ahead * kLoadsPerStage>{});
    });
  }
  __syncthreads();  // the epilogue reuses the LDS
  // A piece of a split tile: unless it is the tile's last to finish, it leaves its partial
  // sums to that one; the last adds them in and stores the tile.
  if (pieces > 1 &&
      !split_fixup<kFragM, kFragN>(acc, piece, pieces, cnt, slots, kSlotFloats,
                                   split_flags, idle, args.status,
                                   args.split_spins))
    return;

  // ---- epilogue ------------------------------------------------------------------------
  // acc[i][j][r] holds tile element (128 wm + 32 i + 8 (r/4) + 4 lk + r%4, 96 wn + 32 j + lr).
  // Each wave stores its own 128 x 96 block, one 32-row slab (fragment row i) at a time,
  // through a private LDS slab; no workgroup barrier is needed.
  if (above) return;
  EpArgs<S> e;
  e.alpha = 1.0f;
  if (g.alpha == kAlphaS) e.alpha = args.scale[lo];
  else if (g.alpha == kAlphaS2) e.alpha = args.scale[lo] * args.scale[lo];
  else if (g.alpha == kAlphaQuarter) e.alpha = sqrtf(sqrtf(args.scale[lo]));
  e.pa = args.pa;
  e.pb = args.pb;
  e.pc = args.pc;
  e.step = d.eta * e.alpha;
  e.C = to_global(static_cast<S*>(C.ptr));
  e.ldc = C.ld;
  e.E = to_global(static_cast<const S*>(g.e >= 0 ? d.buf[g.e].ptr : C.ptr));
  e.lde = g.e >= 0 ? d.buf[g.e].ld : 0;
  const bool xform = kind == kOpXform;
  e.T = xform ? to_global(static_cast<S*>(d.buf[g.c2].ptr)) : e.C;
  e.ldt = xform ? d.buf[g.c2].ld : e.ldc;
  e.rows_out = rows_out;
  e.cols_out = cols_out;
  e.m = rows_out;
  e.d_rows = xform ? C.rows : rows_out;
  e.d_cols = xform ? C.kpad : C.kpad;
  e.t_rows = xform ? d.buf[g.c2].rows : rows_out;
  e.t_cols = xform ? d.buf[g.c2].kpad : C.kpad;
  e.wvec = d.wvec;
  e.wbf16 = d.gram_f32;
  e.r0 = row0 + kWaveRows * wm;
  e.c0 = col0 + kWaveCols * wn;
  e.lane = lane;
  char* slab = (wave < kWaves / 2 ? lds0 : lds1) + (wave % (kWaves / 2)) * kSlabBytes;
  switch (kind) {
    case kOpSyrk: ep_wave<kOpSyrk>(acc, e, slab); break;
    case kOpPoly: ep_wave<kOpPoly>(acc, e, slab); break;
    case kOpXform: ep_wave<kOpXform>(acc, e, slab); break;
    case kOpIdent: ep_wave<kOpIdent>(acc, e, slab); break;
    case kOpUpdate: ep_wave<kOpUpdate>(acc, e, slab); break;
    default: ep_wave<kOpProd>(acc, e, slab); break;
  }

}

// The launch: workgroups [0, dp_tiles) run whole tiles in the XCD-aware order; with a tail
// split the next tail_wgs run one piece each of the last tail_tiles tiles (tile_order.h).
template <typename S>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_wide(GemmArgs args) {
  const int w = int(blockIdx.x);
  int t = 0, piece = 0, pieces = 1;
  int32_t* cnt = nullptr;
  float* slots = nullptr;
  if (w < args.dp_tiles) {
    t = xcd_remap(w, args.dp_tiles);
  } else {
    if (!split_item(args.split_mode, args.tail_tiles, args.tail_wgs, args.split_c, w - args.dp_tiles, t,
                    piece, pieces))
      return;
    cnt = args.split_cnt + 2 * t;
    slots = args.split_slots + int64_t(t) * pieces * kSlotFloats;
    t += args.dp_tiles;
  }
  gemm_wide_tile<S>(args, t, piece, pieces, cnt, slots);
}

}  // namespace

int muon_launch_gemm_wide(const GemmArgs& a, int dtype, void* stream) {
  if (a.grid <= 0) return hipSuccess;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_gemm_wide<uint16_t>, dim3(a.grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm_wide<float>, dim3(a.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// Test hook for host-side checks of the wide tiles: tile t of one output -> (ti[t], tj[t]);
// tri != 0: the tiles of a symmetric rows x rows output on or below the diagonal, else the
// full grid of a rows x cols output.  Returns the tile count.
extern "C" int muon_debug_wide_tile_order(int tri, int rows, int cols, int* ti, int* tj) {
  const int tm = ceil_div_i(rows, kWideM), tn = ceil_div_i(cols, kWideN);
  const int n = tri ? sym_tiles(rows, kWideM, kWideN) : tm * tn;
  if (!ti || !tj) return n;
  for (int t = 0; t < n; ++t) {
    if (tri) sym_decode(t, rows, kWideM, kWideN, ti[t], tj[t]);
    else full_band_decode(t, tm, tn, ti[t], tj[t]);
  }
  return n;
}
