// Grouped MFMA contraction kernel of the Gram Newton-Schulz step for gfx950 (CDNA4).
//
// Every product of the step has the form C = A B^T with both operands stored row-major
// with the contraction index contiguous: the Gram iterates are symmetric (each is a
// polynomial in G0 = X0 X0^T), so B^T = B, and the row form X and the transposed form
// X^T are both kept in HBM.  One launch serves several op groups (a group = one op on a
// contiguous run of same-schedule matrices of one shape bucket; DMuon summary §2.2,
// batching of similar shapes), and every workgroup computes one 256 x 256 output tile
// (128 x 128 in the small-tile build).
//
// Symmetric outputs (DMuon summary §2.2, SYRK-type path over the lower triangle) use the
// lower-triangle tiles only; each computed element (i >= j) is stored at (i, j) and at
// (j, i), so every stored iterate is exactly symmetric.
//
// Main loop: 8 waves of 64 lanes in a 2 x 4 grid, each wave owning 128 x 64 = 4 x 2 blocks
// of 32 x 32 MFMA accumulators (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x2_f32 for
// fp32; fp32 accumulate); the small-tile build has 4 waves in a 2 x 2 grid, 64 x 64 each.  A stage holds kRowBytes of every operand row (64 bf16 or 32
// fp32 with 128-byte rows).  Operands go straight from global memory to LDS
// (global_load_lds_dwordx4: 16 bytes per lane, 1 KB per wave instruction), so no VGPRs
// or LDS-write instructions are spent on staging.  LDS rows are unpadded; the 16-byte
// chunk c of row r sits at chunk position c ^ swz(r).  The LDS serves 16 lanes of a
// 16-byte read per cycle from 64 four-byte banks (256 bytes), and a fragment read has 16
// consecutive lanes on 16 consecutive rows at the same chunk: with 128-byte rows, two
// rows share a 256-byte bank window, so swz(r) = (r / 2) mod 8 puts the 16 rows on 16
// distinct 16-byte bank groups (64-byte rows: four per window, swz(r) = (r / 4) mod 4).  kStages stages form a ring;
// loads run kStages-1 stages ahead of the MFMAs, with one barrier per stage.  Each stage
// is its own __shared__ array and the k loop is unrolled by kStages, so every LDS access
// names its array statically: the compiler can then tell that the loads in flight target
// other stages and does not make the fragment reads wait for them.
//
// Operand rows past the end of an operand are clamped to its last row: they only feed
// output rows or columns that are never stored, and every load stays in bounds.
//
// Epilogue: the accumulators are staged through LDS (bf16 outputs once, transposed; fp32
// ones one half of the tile at a time), so that the epilogue math reads each input once and both the direct store
// (rows of C) and the mirrored/transposed store (rows of C^T) are coalesced.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "muon_internal.h"
#include "split_fixup.h"
#include "tile_order.h"

using namespace muon;

// The library builds this file three times: the 256 x 256 kernel with 2 stages of 128-byte
// rows (muon_launch_gemm); with MUON_GEMM_DEEP 4 stages of 64-byte rows, three k-steps of
// loads in flight instead of one (muon_launch_gemm_deep, the deep-pipeline configuration);
// and with MUON_GEMM_SMALL 128 x 128 tiles run by 4 waves of 64 x 64 with 2 stages of
// 64-byte rows, whose 35 KB of LDS and at most 168 registers a lane let three workgroups
// share a compute unit, one's epilogue overlapping the others' contractions
// (muon_launch_gemm_small, for launches with few tiles or short contractions).
#ifdef MUON_GEMM_DEEP
#define MUON_GEMM_STAGES 4
#define MUON_GEMM_ROW_BYTES 64
#define MUON_LAUNCH_GEMM muon_launch_gemm_deep
#define MUON_GEMM_KERNEL k_gemm_deep
#elif defined(MUON_GEMM_SMALL)
#define MUON_GEMM_TILE 128
#define MUON_GEMM_ROW_BYTES 64
#define MUON_LAUNCH_GEMM muon_launch_gemm_small
#define MUON_GEMM_KERNEL k_gemm_small
#else
#define MUON_LAUNCH_GEMM muon_launch_gemm
#define MUON_GEMM_KERNEL k_gemm
#endif
#ifndef MUON_GEMM_TILE
#define MUON_GEMM_TILE 256
#endif
#ifndef MUON_GEMM_STAGES
#define MUON_GEMM_STAGES 2
#endif
#ifndef MUON_GEMM_ROW_BYTES
#define MUON_GEMM_ROW_BYTES 128
#endif

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kT = MUON_GEMM_TILE;             // output tile edge (256, or 128)
constexpr int kThreads = kT == 256 ? 512 : 256;
constexpr int kWaves = kThreads / 64;
constexpr int kWavesN = kWaves / 2;            // waves along the tile columns (2 along the rows)
constexpr int kWaveRows = kT / 2;              // rows of a wave's block (128, or 64)
constexpr int kWaveCols = kT / kWavesN;        // columns of a wave's block (64)
constexpr int kFragM = kWaveRows / 32;         // 32-row MFMA blocks per wave (4, or 2)
constexpr int kFragN = kWaveCols / 32;         // 32-column MFMA blocks per wave (2)
constexpr int kHalf = kT / 2;                  // rows of one fp32 epilogue half
constexpr int kSuper = (kT / 64) * (kT / 64);  // 64 x 64 super-blocks of the store pass
constexpr int kStages = MUON_GEMM_STAGES;
constexpr int kEpLd = kT / kStages + 1;        // fp32 leading dimension of a staged block
                                               // (odd: strided reads spread over the banks)
constexpr int kRowBytes = MUON_GEMM_ROW_BYTES; // bytes of one operand row per stage
constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row
constexpr int kOperandBytes = kT * kRowBytes;
constexpr int kStageBytes = 2 * kOperandBytes;
constexpr int kRowsPerInst = 1024 / kRowBytes; // rows one wave instruction fills
constexpr int kInstPerOperand = kOperandBytes / 1024 / kWaves;  // per wave per stage
// The epilogue stages a half tile (kHalf rows) in fp32, split by column block across the stage
// arrays: array q holds columns [q kEpW, (q + 1) kEpW) with leading dimension kEpLd.
constexpr int kEpW = kT / kStages;
constexpr int kEpArrBytes = kHalf * kEpLd * 4;
// bf16 outputs of the Gram products and re-anchors are staged once, transposed: T-row c
// (a tile column) holds the 256 tile rows; the T-rows are split evenly over the arrays.
constexpr int kTs = kT + 8;                 // bf16 T-row stride (528 bytes: 16-byte aligned)
constexpr int kTRowsPerArr = kT / kStages;
constexpr int kTArrBytes = kTRowsPerArr * kTs * 2;
constexpr int kMaxAB = kStageBytes > kEpArrBytes ? kStageBytes : kEpArrBytes;
constexpr int kArrBytes = kMaxAB > kTArrBytes ? kMaxAB : kTArrBytes;
static_assert(kRowBytes == 128 || kRowBytes == 64, "row bytes per stage");
static_assert(kStages == 2 || kStages == 4, "stage count (the epilogue splits 256 columns)");
static_assert(kStages * kArrBytes <= 160 * 1024, "LDS budget");
static_assert(kT == 256 || (kT == 128 && kStages == 2 && 3 * (kStages * kArrBytes + 1024) <= 160 * 1024),
              "the 128 x 128 kernel keeps to a third of the LDS (three workgroups per compute unit)");
static_assert(kSuper % kWaves == 0, "whole super-blocks per wave");
static_assert(kInstPerOperand >= 1, "every wave loads part of each operand");
static_assert(kKPad % (kStages * kRowBytes / 4) == 0 && kKPad % (kStages * kRowBytes / 2) == 0,
              "padded contraction dims must hold whole blocks of stages");

// Element offset, within T-row c of the bf16 epilogue's staged tile, of the chunk holding
// tile rows r .. r+7 (r a multiple of 8): chunk r / 8 rotated by 2 ((c / 16) mod 4).  With
// the 528-byte T-row stride, a T-row's chunk q starts at 16-byte bank group (c + q) mod 16.
// The staging writes (32 consecutive T-rows, one chunk) then meet each group twice, the
// minimum for 8-byte writes; the store pass's reads (16 lanes: 8 T-rows 8 apart, two
// adjacent chunks) meet 16 distinct groups.
__device__ __forceinline__ int tile_chunk(int c, int r) {
  return (((r >> 3) + 2 * ((c >> 4) & 3)) & (kT / 8 - 1)) * 8;
}

// First tile of a matrix among this kernel's tiles of its kind (lower-triangle or full).
__device__ __forceinline__ int tile_prefix(const MatDesc& x, bool tri) {
  if constexpr (kT == 128) return tri ? x.small_prefix[0] : x.small_prefix[1];
  else return tri ? x.tri_prefix : x.full_prefix;
}

// Chunk position of 16-byte chunk c in LDS row r is c ^ swz(r) (a bijection on a row).
__device__ __forceinline__ int swz(int r) {
  return kRowBytes == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

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
  if (kind == kOpAffine) return alpha * ((gi == gj ? pa : 0.0f) + pb * to_f(E[int64_t(er) * lde + ec]));
  return x;
}

// One output tile of the launch (logical tile `bid`), or piece `piece` of `pieces` of it when
// the tail split cut its contraction (cnt: the tile's two split counters, slots: its
// `pieces` partial-sum slots).
template <typename S, bool kBuf>
__device__ __forceinline__ void gemm_tile(const GemmArgs& args, const int bid, const int piece,
                                          const int pieces, int32_t* const cnt,
                                          float* const slots) {
  __shared__ __attribute__((aligned(1024))) char lds0[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds2[kStages > 2 ? kArrBytes : 16];
  __shared__ __attribute__((aligned(1024))) char lds3[kStages > 3 ? kArrBytes : 16];
  __shared__ int split_flags[2];  // the tail split's flags (split_fixup), apart from the stages
  // Stage array s, named statically when s is a compile-time constant.
  auto stage_of = [&](auto sc) -> char* {
    constexpr int s = decltype(sc)::value % kStages;
    if constexpr (s == 0) return lds0;
    else if constexpr (s == 1) return lds1;
    else if constexpr (s == 2) return lds2;
    else return lds3;
  };

  // ---- which group, matrix and tile --------------------------------------------------
  GroupArg g = args.g[0];
#pragma unroll
  for (int q = 1; q < kMaxGroups; ++q)
    if (q < args.ngroups && args.g[q].tile_begin <= bid) g = args.g[q];
  const MatDesc* desc = args.desc;
  // The tile's matrix: a division when the group's matrices have equal tile counts, else a
  // binary search over the tile prefixes (one dependent descriptor read per step).
  int lo, t;
  if (g.tpm > 0) {
    const int u = bid - g.tile_begin;
    lo = g.first + u / g.tpm;
    t = u % g.tpm;
  } else {
    const bool tri = g.tri != 0;
    const int v = bid - g.tile_begin + tile_prefix(desc[g.first], tri);
    int hi = g.last - 1;
    lo = g.first;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_prefix(desc[mid], tri) <= v) lo = mid; else hi = mid - 1;
    }
    t = v - tile_prefix(desc[lo], tri);
  }
  const MatDesc& d = desc[lo];

  const BufDesc C = d.buf[g.c];
  const int kind = g.kind;
  const bool ident = kind == kOpIdent || kind == kOpAffine;  // no contraction
  const BufDesc A = ident ? C : d.buf[g.a];
  const BufDesc B = ident ? C : d.buf[g.b];
  const int rows_out = A.rows;
  const int cols_out = B.rows;
  int ti, tj;
  if (g.tri) {
    tri_band_decode(t, (rows_out + kT - 1) / kT, ti, tj);
  } else {
    full_band_decode(t, (rows_out + kT - 1) / kT, (cols_out + kT - 1) / kT, ti, tj);
  }
  const int row0 = ti * kT;
  const int col0 = tj * kT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN;   // 0..1: rows [kWaveRows wm, kWaveRows (wm + 1))
  const int wn = wave % kWavesN;   // cols [kWaveCols wn, kWaveCols (wn + 1))
  const int lr = lane & 31;
  const int lk = lane >> 5;
  // In a diagonal tile the waves of the first half of the rows and the second half of the
  // columns lie strictly above the diagonal: nothing they compute is stored.
  const bool above = g.tri && ti == tj && wm == 0 && wn >= kWavesN / 2;
  const bool idle = above || ident;

  f32x16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- loads: wave `wave` fills rows [wave*R, wave*R + R) of each operand per stage,
  // R = kInstPerOperand * kRowsPerInst, one instruction per kRowsPerInst rows.  Lane l of
  // an instruction writes LDS bytes [16 l, 16 l + 16) of its 1 KB block: row l / kChunks
  // of the block, chunk position l % kChunks, holding global chunk (position ^ swz(row)).
  const int ksteps = ident ? 0 : A.kpad / Mma<S>::kStageK;
  int k0 = 0, k1 = ksteps;  // the k-steps of this piece
  if (pieces > 1) split_range(args.split_mode, args.split_n, ksteps, kSplitUnit, piece, pieces, k0, k1);
  // Operand addresses: with kBuf (every operand of the launch below 2 GB) a buffer resource
  // per operand and one 32-bit byte offset per lane and load (buffer_load_dwordx4 ... lds,
  // about 4 % faster than the FLAT global_load_lds on the layer workload); otherwise 64-bit
  // pointers.  Rows past the end of an operand are clamped to its last row either way.
  const int64_t lda = A.ld * int64_t(sizeof(S));
  const int64_t ldb = B.ld * int64_t(sizeof(S));
  const int lrow = lane / kChunks;
  const int lpos = lane % kChunks;
  const char* a_src[kInstPerOperand];
  const char* b_src[kInstPerOperand];
  uint32_t a_off[kInstPerOperand], b_off[kInstPerOperand];
#pragma unroll
  for (int j = 0; j < kInstPerOperand; ++j) {
    const int r = (wave * kInstPerOperand + j) * kRowsPerInst + lrow;  // tile row
    const int chunk = lpos ^ swz(r);
    const int ra = min(row0 + r, A.rows - 1);
    const int rb = min(col0 + r, B.rows - 1);
    a_off[j] = uint32_t(int64_t(ra) * lda + chunk * 16);
    b_off[j] = uint32_t(int64_t(rb) * ldb + chunk * 16);
    a_src[j] = static_cast<const char*>(A.ptr) + int64_t(ra) * lda + chunk * 16;
    b_src[j] = static_cast<const char*>(B.ptr) + int64_t(rb) * ldb + chunk * 16;
  }
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(A.ptr), (short)0, kBuf ? int(uint32_t(A.rows) * uint32_t(lda)) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(B.ptr), (short)0, kBuf ? int(uint32_t(B.rows) * uint32_t(ldb)) : 0, 0x00020000);
  // Issue the loads of k-step ks into stage array st.
  auto issue = [&](int ks, char* st) {
#pragma unroll
    for (int j = 0; j < kInstPerOperand; ++j) {
      const int blk = (wave * kInstPerOperand + j) * 1024;
      if constexpr (kBuf) {
        const int koff = ks * kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void*)(st + blk), 16, a_off[j], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_void*)(st + kOperandBytes + blk), 16, b_off[j],
                                                 koff, 0, 0);
      } else {
        const int64_t koff = int64_t(ks) * kRowBytes;
        __builtin_amdgcn_global_load_lds(a_src[j] + koff, (lds_void*)(st + blk), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(b_src[j] + koff, (lds_void*)(st + kOperandBytes + blk), 16, 0, 0);
      }
    }
  };
  constexpr int kLoadsPerStage = 2 * kInstPerOperand;
  // Prologue: stages 0 .. kStages-2 in flight.
  static_for<0, kStages - 1>([&](auto sc) {
    if (k0 + sc.value < k1) issue(k0 + sc.value, stage_of(sc));
  });

  // Fragment rows of this lane (+ 32 i for A, + 32 j for B).
  const int a_row = wm * kWaveRows + lr;
  const int b_row = wn * kWaveCols + lr;
  constexpr int kKK = kRowBytes / 32;  // MFMA k-blocks per step
  // Fragments of k-block kk (16-byte chunk 2 kk + lk of the lane's rows) from stage st.
  auto load_frags = [&](const char* st, int kk, uint4* fa, uint4* fb) {
    const int c = 2 * kk + lk;
#pragma unroll
    for (int i = 0; i < kFragM; ++i) {
      const int r = a_row + 32 * i;
      fa[i] = *reinterpret_cast<const uint4*>(st + r * kRowBytes + ((c ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < kFragN; ++j) {
      const int r = b_row + 32 * j;
      fb[j] = *reinterpret_cast<const uint4*>(st + kOperandBytes + r * kRowBytes + ((c ^ swz(r)) << 4));
    }
  };
  // One k-step: wait until this wave's loads of stage ks landed (at most `pending` newer
  // loads remain), barrier, issue the loads kStages-1 steps ahead, run the MFMAs.
  auto kstep = [&](int ks, auto sc, auto pending) {
    wait_vm<decltype(pending)::value>();
    stage_barrier();  // all waves' loads of stage ks landed; stage ks-1 is free again
    if (ks + kStages - 1 < k1)
      issue(ks + kStages - 1, stage_of(std::integral_constant<int, decltype(sc)::value + kStages - 1>{}));
    if (idle) return;
    const char* st = stage_of(sc);
    // Scheduling hint for this MFMA block: the compiler then issues the stage's fragment
    // reads early, one between consecutive MFMAs, instead of four or two ahead of each
    // group with a wait on each; measured 2-3 % faster per step, no spills.
    __builtin_amdgcn_iglp_opt(1);
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      uint4 fa[kFragM], fb[kFragN];
      load_frags(st, kk, fa, fb);
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) Mma<S>::step(fa[i], fb[j], acc[i][j]);
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
  // acc[i][j][r] holds tile element (kWaveRows wm + 32 i + 8 (r/4) + 4 lk + r%4,
  // kWaveCols wn + 32 j + lr).
  float alpha = 1.0f;
  if (g.alpha == kAlphaS) alpha = args.scale[lo];
  else if (g.alpha == kAlphaS2) alpha = args.scale[lo] * args.scale[lo];
  else if (g.alpha == kAlphaQuarter) alpha = sqrtf(sqrtf(args.scale[lo]));
  const gptr<S> Cp = to_global(static_cast<S*>(C.ptr));
  const int64_t ldc = C.ld;
  const gptr<const S> E = to_global(static_cast<const S*>(g.e >= 0 ? d.buf[g.e].ptr : C.ptr));
  const int64_t lde = g.e >= 0 ? d.buf[g.e].ld : 0;
  const float pa = args.pa, pb = args.pb, pc = args.pc;
  const int m = rows_out;    // symmetric outputs: valid rows/cols
  const int cstore = C.kpad; // symmetric outputs: stored columns (zero beyond m)

  // bf16 Gram products and re-anchors: each value is formed once, in registers, from its
  // accumulator (and, for the polynomial, the iterate read transposed: it is symmetric),
  // rounded to bf16 and staged transposed in LDS; then two copy passes store the rows of
  // C (direct) and of C^T (mirror or transposed output) with 16-byte stores.
  if constexpr (sizeof(S) == 2) {
    if (kind != kOpUpdate) {
      // T-row c holds tile column c, in chunks of 8 rows placed by tile_chunk.
      auto t_chunk = [&](int c, int r) -> uint16_t* {
        const int q = c / kTRowsPerArr;
        char* base = q == 0 ? lds0 : q == 1 ? lds1 : q == 2 ? lds2 : lds3;
        return reinterpret_cast<uint16_t*>(base) + (c % kTRowsPerArr) * kTs + tile_chunk(c, r);
      };
      const bool xform = kind == kOpXform;
      // Stage the wave's values; K is the op kind as a compile-time constant.
      auto stage = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
#pragma unroll
        for (int i = 0; i < kFragM; ++i) {
          u32x2 e4[kFragN][4];
          if constexpr (K == kOpPoly || K == kOpAffine) {
#pragma unroll
            for (int j = 0; j < kFragN; ++j)
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) {
                const int gi0 = row0 + kWaveRows * wm + 32 * i + 8 * r4 + 4 * lk;
                const int gj = col0 + kWaveCols * wn + 32 * j + lr;
                e4[j][r4] = u32x2{0u, 0u};
                if (gj < m && gi0 < m) e4[j][r4] = *(gptr<const u32x2>)(E + int64_t(gj) * lde + gi0);
              }
          }
#pragma unroll
          for (int j = 0; j < kFragN; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int lrow = kWaveRows * wm + 32 * i + 8 * r4 + 4 * lk;  // 4 rows lrow .. lrow+3
              const int lcol = kWaveCols * wn + 32 * j + lr;
              const int gi0 = row0 + lrow, gj = col0 + lcol;
              uint16_t o[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int gi = gi0 + q;
                const float x = acc[i][j][4 * r4 + q];
                float val;
                if constexpr (K == kOpXform) {
                  val = (gi < rows_out && gj < cols_out) ? alpha * x : 0.0f;
                } else {
                  const bool in = gi < m && gj < m;
                  if constexpr (K == kOpSyrk) val = in ? alpha * x : 0.0f;
                  else if constexpr (K == kOpPoly)
                    val = in ? (gi == gj ? pa : 0.0f) +
                                   pb * to_f(reinterpret_cast<const uint16_t*>(&e4[j][r4])[q]) + pc * x
                             : 0.0f;
                  else if constexpr (K == kOpIdent) val = (in && gi == gj) ? 1.0f : 0.0f;
                  else if constexpr (K == kOpAffine)
                    val = in ? alpha * ((gi == gj ? pa : 0.0f) +
                                        pb * to_f(reinterpret_cast<const uint16_t*>(&e4[j][r4])[q]))
                             : 0.0f;
                  else val = in ? x : 0.0f;
                }
                o[q] = from_f(val, static_cast<uint16_t*>(nullptr));
              }
              *reinterpret_cast<uint2*>(t_chunk(lcol, lrow & ~7) + (lrow & 7)) = *reinterpret_cast<const uint2*>(o);
            }
        }
      };
      if (!above) {
        switch (kind) {
          case kOpSyrk: stage(std::integral_constant<int, kOpSyrk>{}); break;
          case kOpPoly: stage(std::integral_constant<int, kOpPoly>{}); break;
          case kOpXform: stage(std::integral_constant<int, kOpXform>{}); break;
          case kOpIdent: stage(std::integral_constant<int, kOpIdent>{}); break;
          case kOpAffine: stage(std::integral_constant<int, kOpAffine>{}); break;
          default: stage(std::integral_constant<int, kOpProd>{}); break;
        }
      }
      __syncthreads();
      // Store pass, in 8 x 8 blocks.  Lane l of a wave takes block row 8 sr + (l >> 3) and
      // block column 8 sc + (l & 7) of one of the wave's two 64 x 64 super-blocks (sr, sc).
      // Its eight 16-byte LDS reads are the block's columns: runs of 8 elements of rows of
      // C^T (the mirror, or an xform's transposed output); an 8 x 8 transpose in registers
      // gives the runs of rows of C (direct).  Eight consecutive lanes cover 128 contiguous
      // bytes of one output row either way, so each store instruction writes whole lines.
      // Every output here is a workspace buffer whose stored width (kpad) is a multiple of
      // kKPad, so a block's 8 columns are stored whole or not at all.  On a symmetric output
      // a block lies strictly below the diagonal (both sides stored), on it (its lower half
      // and the mirror of that half, as one symmetric block from the direct side), or
      // strictly above (nothing stored).
      const bool tpass = !xform || g.c2 >= 0;  // an xform without a transposed output skips it
      const BufDesc T2 = (xform && g.c2 >= 0) ? d.buf[g.c2] : C;
      const gptr<S> Tp = xform ? to_global(static_cast<S*>(T2.ptr)) : Cp;
      const int64_t ldt = xform ? T2.ld : ldc;
      const int t_rows = xform ? T2.rows : m;          // valid rows of the transposed side
      const int t_cols = xform ? T2.kpad : cstore;     // its stored columns
      const int d_rows = xform ? C.rows : m;
      const int d_cols = xform ? C.kpad : cstore;
#pragma unroll
      for (int sb = 0; sb < kSuper / kWaves; ++sb) {
        const int sblk = wave + kWaves * sb;  // super-block 0 .. kSuper - 1
        const int r = 64 * (sblk / (kT / 64)) + 8 * (lane >> 3);
        const int c = 64 * (sblk % (kT / 64)) + 8 * (lane & 7);
        const int gi = row0 + r, gj = col0 + c;
        if (!xform && gi < gj) continue;
        const bool diag = !xform && gi == gj;
        u32x4 blk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) blk[e] = *reinterpret_cast<const u32x4*>(t_chunk(c + e, r));
        // Element (r + q, c + e) of the tile is half (q & 1) of dword q / 2 of blk[e].
        auto elem = [&](int q, int e) -> uint32_t {
          const uint32_t w = blk[e][q >> 1];
          return (q & 1) ? (w >> 16) : (w & 0xffffu);
        };
        // Transposed side: row gj + e gets tile rows r .. r+7 of column c + e.
        if (tpass && !diag && gi < t_cols) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gj + e < t_rows) store8(Tp + int64_t(gj + e) * ldt + gi, __builtin_bit_cast(Vec8<S>, blk[e]));
        }
        // Direct side: row gi + q gets tile columns c .. c+7 of row r + q; on a diagonal
        // block the elements above the diagonal are the mirrors, (r + e, c + q).
        if (gj < d_cols) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (gi + q >= d_rows) continue;
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int e0 = 2 * k, e1 = 2 * k + 1;
              const uint32_t lo = (diag && e0 > q) ? elem(e0, q) : elem(q, e0);
              const uint32_t hi = (diag && e1 > q) ? elem(e1, q) : elem(q, e1);
              o[k] = lo | (hi << 16);
            }
            store8(Cp + int64_t(gi + q) * ldc + gj, __builtin_bit_cast(Vec8<S>, o));
          }
        }
      }
      return;
    }
  }

  // fp32 path (the update, and every op of the fp32 kernel): the accumulators are staged in
  // fp32, one half (kHalf rows) at a time, split by column block across the stage arrays.
  auto ep_at = [&](int rr, int cc) -> float& {
    const int q = cc / kEpW;
    char* base = q == 0 ? lds0 : q == 1 ? lds1 : q == 2 ? lds2 : lds3;
    return reinterpret_cast<float*>(base)[rr * kEpLd + cc % kEpW];
  };
  // Chunks of 8 consecutive elements.  Direct passes: 8 columns of one row, consecutive lanes
  // on consecutive chunks of a row.  Mirror passes: 8 rows of one column, written as 8
  // consecutive columns of the transposed output, consecutive lanes on consecutive row
  // chunks.  Full chunks use one 16- or 32-byte access; chunks that cross the diagonal or an
  // edge fall back to single elements.
  constexpr int kRowChunks = kT / 8;       // chunks per row of a half
  constexpr int kColChunks = kHalf / 8;    // chunks per column of a half
  constexpr int kChunksHalf = kHalf * kRowChunks;
  // Accumulators of rows [kHalf half, kHalf (half + 1)) into the stage arrays.
  auto stage_half = [&](int half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            ep_at(32 * i + 8 * (r >> 2) + 4 * lk + (r & 3), kWaveCols * wn + 32 * j + lr) = acc[i][j][r];
    }
  };
  if (kind == kOpUpdate) {  // W -= eta * alpha * (A B^T)
    const float step = d.eta * alpha;
    // W's element type Wt: S, or bf16 for a bf16 matrix whose Gram iteration ran in fp32.
    auto update = [&](auto wt) {
      using Wt = decltype(wt);
      const gptr<Wt> Wp = to_global(static_cast<Wt*>(C.ptr));
      constexpr int kPer = kChunksHalf / kThreads;  // chunks per thread and half
      constexpr int kBatch = sizeof(Wt) == 2 ? kPer : kPer / 2;  // W chunks held at once
      static_assert(kChunksHalf % kThreads == 0 && kPer % kBatch == 0, "whole chunks per thread");
      Vec8<Wt> w[kBatch];
      auto chunk = [&](int u, int& rr, int& cc) {  // chunk u of this thread in a half
        const int idx = tid + u * kThreads;
        rr = idx / kRowChunks;
        cc = (idx % kRowChunks) * 8;
      };
      auto load_batch = [&](int half, int b) {
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
          int rr, cc;
          chunk(b + v, rr, cc);
          const int gi = row0 + half * kHalf + rr, gj = col0 + cc;
          if (gi < rows_out && d.wvec && gj + 7 < cols_out) load8<Wt>(Wp + int64_t(gi) * ldc + gj, w[v]);
        }
      };
      for (int half = 0; half < 2; ++half) {
        // The half's first W chunks are requested before its accumulators are staged, so
        // their latency overlaps the staging; each batch is one load round trip.
        load_batch(half, 0);
        stage_half(half);
        __syncthreads();
#pragma unroll
        for (int b = 0; b < kPer; b += kBatch) {
          if (b > 0) load_batch(half, b);
#pragma unroll
          for (int v = 0; v < kBatch; ++v) {
            int rr, cc;
            chunk(b + v, rr, cc);
            const int gi = row0 + half * kHalf + rr, gj = col0 + cc;
            if (gi >= rows_out || gj >= cols_out) continue;
            const gptr<Wt> p = Wp + int64_t(gi) * ldc + gj;
            if (d.wvec && gj + 7 < cols_out) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                w[v].v[e] = from_f(fmaf(-step, ep_at(rr, cc + e), to_f(w[v].v[e])), static_cast<Wt*>(nullptr));
              store8(p, w[v]);
            } else {
              for (int e = 0; e < 8 && gj + e < cols_out; ++e)
                p[e] = from_f(fmaf(-step, ep_at(rr, cc + e), to_f(p[e])), static_cast<Wt*>(nullptr));
            }
          }
        }
        __syncthreads();
      }
    };
    if (sizeof(S) == 4 && d.gram_f32) update(uint16_t());
    else update(S());
    return;
  }
  for (int half = 0; half < 2; ++half) {
    const int hr0 = row0 + half * kHalf;  // first row of this half
    if (!ident) {
      stage_half(half);
      __syncthreads();
    }
    if (g.tri) {
      for (int idx = tid; idx < kChunksHalf; idx += kThreads) {
        const int rr = idx / kRowChunks, cc = (idx % kRowChunks) * 8;
        const int gi = hr0 + rr, gj = col0 + cc;
        if (gi >= m || gi < gj) continue;  // row invalid, or the chunk lies above the diagonal
        if (gi >= gj + 7 && gj + 7 < m) {
          Vec8<S> e8, out;
          if (kind == kOpPoly || kind == kOpAffine) load8<S>(E + int64_t(gi) * lde + gj, e8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = ident ? 0.0f : ep_at(rr, cc + e);
            float val;
            if (kind == kOpSyrk) val = alpha * x;
            else if (kind == kOpPoly) val = (gi == gj + e ? pa : 0.0f) + pb * to_f(e8.v[e]) + pc * x;
            else if (kind == kOpIdent) val = gi == gj + e ? 1.0f : 0.0f;
            else if (kind == kOpAffine) val = alpha * ((gi == gj + e ? pa : 0.0f) + pb * to_f(e8.v[e]));
            else val = x;
            out.v[e] = from_f(val, static_cast<S*>(nullptr));
          }
          store8(Cp + int64_t(gi) * ldc + gj, out);
        } else {
          for (int e = 0; e < 8; ++e) {
            const int gje = gj + e;
            if (gi < gje || gje >= cstore) continue;
            const float x = ident ? 0.0f : ep_at(rr, cc + e);
            Cp[int64_t(gi) * ldc + gje] =
                from_f(tri_value<S>(kind, gi, gje, m, x, alpha, E, lde, gi, gje, pa, pb, pc), static_cast<S*>(nullptr));
          }
        }
      }
      for (int idx = tid; idx < kChunksHalf; idx += kThreads) {
        const int rr = (idx % kColChunks) * 8, cc = idx / kColChunks;
        const int gi = hr0 + rr, gj = col0 + cc;
        if (gj >= m || gi + 7 <= gj) continue;  // row of C invalid, or chunk on/above diagonal
        if (gi > gj && gi + 7 < m) {
          Vec8<S> e8, out;
          if (kind == kOpPoly || kind == kOpAffine) load8<S>(E + int64_t(gj) * lde + gi, e8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = ident ? 0.0f : ep_at(rr + e, cc);
            float val;
            if (kind == kOpSyrk) val = alpha * x;
            else if (kind == kOpPoly) val = pb * to_f(e8.v[e]) + pc * x;  // off-diagonal: no pa
            else if (kind == kOpIdent) val = 0.0f;
            else if (kind == kOpAffine) val = alpha * pb * to_f(e8.v[e]);
            else val = x;
            out.v[e] = from_f(val, static_cast<S*>(nullptr));
          }
          store8(Cp + int64_t(gj) * ldc + gi, out);
        } else {
          for (int e = 0; e < 8; ++e) {
            const int gie = gi + e;
            if (gie <= gj || gie >= cstore) continue;
            const float x = ident ? 0.0f : ep_at(rr + e, cc);
            Cp[int64_t(gj) * ldc + gie] =
                from_f(tri_value<S>(kind, gie, gj, m, x, alpha, E, lde, gj, gie, pa, pb, pc), static_cast<S*>(nullptr));
          }
        }
      }
    } else {  // kOpXform
      // Row form C (rows < C.rows, columns < C.kpad, zero beyond cols_out) and its
      // transpose C2 (rows < C2.rows, columns < C2.kpad, zero beyond rows_out).  Both
      // leading dimensions are multiples of 8, so chunks never straddle the padding edge.
      const BufDesc C2 = g.c2 >= 0 ? d.buf[g.c2] : C;
      const gptr<S> C2p = to_global(static_cast<S*>(C2.ptr));
      for (int idx = tid; idx < kChunksHalf; idx += kThreads) {
        const int rr = idx / kRowChunks, cc = (idx % kRowChunks) * 8;
        const int gi = hr0 + rr, gj = col0 + cc;
        if (gi >= C.rows || gj >= C.kpad) continue;
        Vec8<S> out;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          out.v[e] = from_f(gj + e < cols_out ? alpha * ep_at(rr, cc + e) : 0.0f, static_cast<S*>(nullptr));
        store8(Cp + int64_t(gi) * ldc + gj, out);
      }
      for (int idx = tid; g.c2 >= 0 && idx < kChunksHalf; idx += kThreads) {
        const int rr = (idx % kColChunks) * 8, cc = idx / kColChunks;
        const int gi = hr0 + rr, gj = col0 + cc;
        if (gj >= C2.rows || gi >= C2.kpad) continue;
        Vec8<S> out;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          out.v[e] = from_f(gi + e < rows_out ? alpha * ep_at(rr + e, cc) : 0.0f, static_cast<S*>(nullptr));
        store8(C2p + int64_t(gj) * C2.ld + gi, out);
      }
    }
    if (!ident) __syncthreads();
  }
}

// The launch: workgroups [0, dp_tiles) run whole tiles in the XCD-aware order; with a tail
// split the next tail_wgs run one piece each of the last tail_tiles tiles (tile_order.h).
// Registers: the 256 x 256 kernel's 8 waves run two per SIMD (256 a lane); three workgroups
// of the 128 x 128 kernel's 4 waves run three per SIMD (168 a lane).
template <typename S, bool kBuf>
__global__ __launch_bounds__(kThreads, kT == 256 ? 1 : 3) void MUON_GEMM_KERNEL(GemmArgs args) {
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
  gemm_tile<S, kBuf>(args, t, piece, pieces, cnt, slots);
}

}  // namespace

int MUON_LAUNCH_GEMM(const GemmArgs& a, int dtype, void* stream) {
  if (a.grid <= 0) return hipSuccess;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == kBF16 && a.buf32)
    hipLaunchKernelGGL((MUON_GEMM_KERNEL<uint16_t, true>), dim3(a.grid), dim3(kThreads), 0, s, a);
  else if (dtype == kBF16)
    hipLaunchKernelGGL((MUON_GEMM_KERNEL<uint16_t, false>), dim3(a.grid), dim3(kThreads), 0, s, a);
  else if (a.buf32)
    hipLaunchKernelGGL((MUON_GEMM_KERNEL<float, true>), dim3(a.grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((MUON_GEMM_KERNEL<float, false>), dim3(a.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

#if !defined(MUON_GEMM_DEEP) && !defined(MUON_GEMM_SMALL)
// Test hooks for host-side checks of tile_order.h.
extern "C" int muon_debug_xcd_remap(int total, int* out) {
  for (int w = 0; w < total; ++w) out[w] = xcd_remap(w, total);
  return total;
}

extern "C" int muon_debug_tile_order(int tri, int tm, int tn, int* ti, int* tj) {
  const int n = tri ? tm * (tm + 1) / 2 : tm * tn;
  for (int t = 0; t < n; ++t) {
    if (tri) tri_band_decode(t, tm, ti[t], tj[t]);
    else full_band_decode(t, tm, tn, ti[t], tj[t]);
  }
  return n;
}
#endif  // MUON_GEMM_DEEP
