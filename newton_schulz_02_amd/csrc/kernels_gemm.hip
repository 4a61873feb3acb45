// Grouped MFMA contraction kernel of the Gram Newton-Schulz step for gfx950 (CDNA4).
//
// Every product of the step has the form C = A B^T with both operands stored row-major
// with the contraction index contiguous: the Gram iterates are symmetric (each is a
// polynomial in G0 = X0 X0^T), so B^T = B, and the row form X and the transposed form
// X^T are both kept in HBM.  One launch serves several op groups (a group = one op on a
// contiguous run of same-schedule matrices of one shape bucket; DMuon summary §2.2,
// batching of similar shapes), and every workgroup computes one 256 x 256 output tile.
//
// Symmetric outputs (DMuon summary §2.2, SYRK-type path over the lower triangle) use the
// lower-triangle tiles only; each computed element (i >= j) is stored at (i, j) and at
// (j, i), so every stored iterate is exactly symmetric.
//
// Tile: 256 x 256 x 64 (bf16) or 256 x 256 x 32 (fp32) per LDS stage, 8 waves of 64 lanes
// in a 2 x 4 grid, each wave owning 128 x 64 = 4 x 2 blocks of 32 x 32 MFMA accumulators
// (v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x2_f32, fp32 accumulate).  Operand rows
// are 128 bytes per stage; LDS rows are padded to 144 bytes so the 16-byte fragment reads
// of 8 consecutive rows hit distinct bank groups.  Two LDS stages with a register
// prefetch of the next stage overlap global loads with the MFMA work.
//
// Epilogue: the accumulators are staged through LDS as fp32, one 128-row half of the tile
// at a time, so that the epilogue math reads each input once and both the direct store
// (rows of C) and the mirrored/transposed store (rows of C^T) are coalesced.
#include <hip/hip_runtime.h>

#include "muon_internal.h"

using namespace muon;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kWavesN = 4;                 // waves along the tile columns
constexpr int kFragN = kTile / kWavesN / 32;  // 32-wide blocks per wave along N (2)
constexpr int kEpLd = kTile + 4;           // fp32 leading dimension of the staged half tile
constexpr int kRowBytes = 128;             // bytes of one operand row per LDS stage
constexpr int kLdsRow = kRowBytes + 16;    // padded LDS row
constexpr int kOperandBytes = kTile * kLdsRow;
constexpr int kStageBytes = 2 * kOperandBytes;
constexpr int kChunksPerThread = kTile * kRowBytes / 16 / kThreads;  // 4
constexpr int kChunkRows = kThreads / (kRowBytes / 16);               // 64 rows per chunk slab
static_assert(128 * kEpLd * 4 <= 2 * kStageBytes, "staged half tile must fit in LDS");

__device__ __forceinline__ float to_f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ float to_f(float f) { return f; }
__device__ __forceinline__ uint16_t from_f(float f, uint16_t*) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float from_f(float f, float*) { return f; }

// Lower-triangle tile index t -> (ti, tj), ti >= tj, row-major over the triangle.
__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = int((sqrtf(8.0f * float(t) + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// MFMA step over one 16-byte fragment per operand.
template <typename S>
struct Mma;

template <>
struct Mma<uint16_t> {
  static constexpr int kStageK = 64;   // k elements per stage
  __device__ __forceinline__ static void step(const uint4& a, const uint4& b, f32x16& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int kStageK = 32;
  // The fragment holds 4 consecutive k values per lane; MFMA e contracts over element e
  // of both operands (A and B use the same k map, so the sum covers all 8 k values).
  __device__ __forceinline__ static void step(const uint4& a, const uint4& b, f32x16& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Value of the symmetric-output epilogues at (gi, gj); x is the accumulated product.  E is
// read at (er, ec), which is (gi, gj) or its mirror: stored iterates are exactly symmetric.
template <typename S>
__device__ __forceinline__ float tri_value(int kind, int gi, int gj, int m, float x, float alpha,
                                           const S* E, int64_t lde, int er, int ec, float pa,
                                           float pb, float pc) {
  if (gi >= m || gj >= m) return 0.0f;
  if (kind == kOpSyrk) return alpha * x;
  if (kind == kOpPoly) return (gi == gj ? pa : 0.0f) + pb * to_f(E[int64_t(er) * lde + ec]) + pc * x;
  if (kind == kOpIdent) return gi == gj ? 1.0f : 0.0f;
  return x;
}

template <typename S>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];

  // ---- which group, matrix and tile --------------------------------------------------
  const int bid = int(blockIdx.x);
  GroupArg g = args.g[0];
#pragma unroll
  for (int q = 1; q < kMaxGroups; ++q)
    if (q < args.ngroups && args.g[q].tile_begin <= bid) g = args.g[q];
  const MatDesc* desc = args.desc;
  const int v = bid - g.tile_begin + (g.tri ? desc[g.first].tri_prefix : desc[g.first].full_prefix);
  int lo = g.first, hi = g.last - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int pre = g.tri ? desc[mid].tri_prefix : desc[mid].full_prefix;
    if (pre <= v) lo = mid; else hi = mid - 1;
  }
  const MatDesc& d = desc[lo];
  const int t = v - (g.tri ? d.tri_prefix : d.full_prefix);

  const BufDesc C = d.buf[g.c];
  const int kind = g.kind;
  const bool ident = kind == kOpIdent;
  const BufDesc A = ident ? C : d.buf[g.a];
  const BufDesc B = ident ? C : d.buf[g.b];
  const int rows_out = A.rows;
  const int cols_out = B.rows;
  int ti, tj;
  if (g.tri) {
    tri_decode(t, ti, tj);
  } else {
    const int tn = (cols_out + kTile - 1) / kTile;
    ti = t / tn;
    tj = t % tn;
  }
  const int row0 = ti * kTile;
  const int col0 = tj * kTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWavesN;   // 0..1: rows [128 wm, 128 wm + 128)
  const int wn = wave % kWavesN;   // 0..3: cols [64 wn, 64 wn + 64)
  const int lr = lane & 31;
  const int lk = lane >> 5;
  // In a diagonal tile the waves with rows [0,128) and columns [128,256) lie strictly above
  // the diagonal: nothing they compute is stored.
  const bool idle = (g.tri && ti == tj && wm == 0 && wn >= 2) || ident;

  f32x16 acc[4][kFragN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- main loop -----------------------------------------------------------------------
  const int ksteps = ident ? 0 : A.kpad / Mma<S>::kStageK;
  const char* Ab = static_cast<const char*>(A.ptr);
  const char* Bb = static_cast<const char*>(B.ptr);
  const int64_t lda = A.ld * int64_t(sizeof(S));
  const int64_t ldb = B.ld * int64_t(sizeof(S));
  const int crow = tid >> 3;         // chunk row within a 64-row slab
  const int cbyte = (tid & 7) * 16;  // chunk byte within the row
  // Chunk q of this thread is row (crow + 64q) of the tile; rows past the operand read 0.
  const int a_lim = A.rows - row0 - crow;
  const int b_lim = B.rows - col0 - crow;
  const char* a_base = Ab + int64_t(row0 + crow) * lda + cbyte;
  const char* b_base = Bb + int64_t(col0 + crow) * ldb + cbyte;
  const int64_t a_step = kChunkRows * lda;
  const int64_t b_step = kChunkRows * ldb;
  uint4 ra[kChunksPerThread], rb[kChunksPerThread];
  auto gload = [&](int ks) {
    const int64_t koff = int64_t(ks) * kRowBytes;
#pragma unroll
    for (int q = 0; q < kChunksPerThread; ++q) {
      ra[q] = kChunkRows * q < a_lim ? *reinterpret_cast<const uint4*>(a_base + q * a_step + koff)
                                     : make_uint4(0, 0, 0, 0);
      rb[q] = kChunkRows * q < b_lim ? *reinterpret_cast<const uint4*>(b_base + q * b_step + koff)
                                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    char* As = smem + stage * kStageBytes;
    char* Bs = As + kOperandBytes;
#pragma unroll
    for (int q = 0; q < kChunksPerThread; ++q) {
      const int rr = crow + kChunkRows * q;
      *reinterpret_cast<uint4*>(As + rr * kLdsRow + cbyte) = ra[q];
      *reinterpret_cast<uint4*>(Bs + rr * kLdsRow + cbyte) = rb[q];
    }
  };

  if (ksteps > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int ks = 0; ks < ksteps; ++ks) {
    const int stage = ks & 1;
    if (ks + 1 < ksteps) gload(ks + 1);
    if (!idle) {
      const char* As = smem + stage * kStageBytes + (wm * 128 + lr) * kLdsRow + lk * 16;
      const char* Bs = smem + stage * kStageBytes + kOperandBytes + (wn * 64 + lr) * kLdsRow + lk * 16;
#pragma unroll
      for (int kk = 0; kk < kRowBytes / 32; ++kk) {
        uint4 fa[4], fb[kFragN];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[i] = *reinterpret_cast<const uint4*>(As + i * 32 * kLdsRow + kk * 32);
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
          fb[j] = *reinterpret_cast<const uint4*>(Bs + j * 32 * kLdsRow + kk * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < kFragN; ++j) Mma<S>::step(fa[i], fb[j], acc[i][j]);
      }
    }
    if (ks + 1 < ksteps) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------------
  // acc[i][j][r] holds tile element (128 wm + 32 i + 8 (r/4) + 4 lk + r%4, 64 wn + 32 j + lr).
  float alpha = 1.0f;
  if (g.alpha == kAlphaS) alpha = args.scale[lo];
  else if (g.alpha == kAlphaS2) alpha = args.scale[lo] * args.scale[lo];
  float* ep = reinterpret_cast<float*>(smem);
  S* Cp = static_cast<S*>(C.ptr);
  const int64_t ldc = C.ld;
  const S* E = g.e >= 0 ? static_cast<const S*>(d.buf[g.e].ptr) : nullptr;
  const int64_t lde = g.e >= 0 ? d.buf[g.e].ld : 0;
  const float pa = args.pa, pb = args.pb, pc = args.pc;
  const int m = rows_out;   // symmetric outputs: valid rows/cols
  const int cstore = C.kpad; // symmetric outputs: stored columns (zero beyond m)

  for (int half = 0; half < 2; ++half) {
    const int hr0 = row0 + half * 128;  // first row of this half
    if (!ident) {
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < kFragN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              ep[(32 * i + 8 * (r >> 2) + 4 * lk + (r & 3)) * kEpLd + 64 * wn + 32 * j + lr] =
                  acc[i][j][r];
      }
      __syncthreads();
    }
    if (g.tri) {
      // Direct store of the elements on or below the diagonal: row hr0 + rr, 4 columns.
      for (int idx = tid; idx < 128 * (kTile / 4); idx += kThreads) {
        const int rr = idx / (kTile / 4);
        const int cc = (idx % (kTile / 4)) * 4;
        const int gi = hr0 + rr;
        if (gi >= m) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gj = col0 + cc + e;
          if (gi < gj || gj >= cstore) continue;
          const float x = ident ? 0.0f : ep[rr * kEpLd + cc + e];
          Cp[int64_t(gi) * ldc + gj] =
              from_f(tri_value(kind, gi, gj, m, x, alpha, E, lde, gi, gj, pa, pb, pc),
                     static_cast<S*>(nullptr));
        }
      }
      // Mirrored store of the elements strictly below the diagonal: row gj of C gets
      // columns hr0 + rr .. hr0 + rr + 3.
      for (int idx = tid; idx < kTile * 32; idx += kThreads) {
        const int cc = idx / 32;          // tile column -> row of C
        const int rr = (idx % 32) * 4;    // 4 consecutive tile rows -> columns of C
        const int gj = col0 + cc;
        if (gj >= m) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = hr0 + rr + e;
          if (gi <= gj || gi >= cstore) continue;
          const float x = ident ? 0.0f : ep[(rr + e) * kEpLd + cc];
          Cp[int64_t(gj) * ldc + gi] =
              from_f(tri_value(kind, gi, gj, m, x, alpha, E, lde, gj, gi, pa, pb, pc),
                     static_cast<S*>(nullptr));
        }
      }
    } else if (kind == kOpXform) {
      const BufDesc C2 = d.buf[g.c2];
      S* C2p = static_cast<S*>(C2.ptr);
      for (int idx = tid; idx < 128 * (kTile / 4); idx += kThreads) {
        const int rr = idx / (kTile / 4);
        const int cc = (idx % (kTile / 4)) * 4;
        const int gi = hr0 + rr;
        if (gi >= C.rows) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gj = col0 + cc + e;
          if (gj >= C.kpad) continue;
          Cp[int64_t(gi) * ldc + gj] =
              from_f(gj < cols_out ? alpha * ep[rr * kEpLd + cc + e] : 0.0f, static_cast<S*>(nullptr));
        }
      }
      for (int idx = tid; idx < kTile * 32; idx += kThreads) {
        const int cc = idx / 32;
        const int rr = (idx % 32) * 4;
        const int gj = col0 + cc;
        if (gj >= C2.rows) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = hr0 + rr + e;
          if (gi >= C2.kpad) continue;
          C2p[int64_t(gj) * C2.ld + gi] =
              from_f(gi < rows_out ? alpha * ep[(rr + e) * kEpLd + cc] : 0.0f, static_cast<S*>(nullptr));
        }
      }
    } else {  // kOpUpdate: W -= eta * alpha * (A B^T)
      const float step = d.eta * alpha;
      for (int idx = tid; idx < 128 * (kTile / 4); idx += kThreads) {
        const int rr = idx / (kTile / 4);
        const int cc = (idx % (kTile / 4)) * 4;
        const int gi = hr0 + rr;
        if (gi >= rows_out) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gj = col0 + cc + e;
          if (gj >= cols_out) continue;
          S* p = Cp + int64_t(gi) * ldc + gj;
          *p = from_f(fmaf(-step, ep[rr * kEpLd + cc + e], to_f(*p)), static_cast<S*>(nullptr));
        }
      }
    }
    if (!ident) __syncthreads();
  }
}

}  // namespace

int muon_launch_gemm(const GemmArgs& a, int dtype, void* stream) {
  if (a.total_tiles <= 0) return hipSuccess;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_gemm<uint16_t>, dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm<float>, dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
