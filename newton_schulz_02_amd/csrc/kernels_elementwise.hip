// HBM-bound kernels of the Muon step for gfx950:
//   k_momentum  M <- beta*M + G (fp32 math, stored in M's dtype), per-tile partial sums of
//               M'^2 (wave64 shuffle reduction), and the zero-padded row / transposed
//               copies that the MFMA phase reads (transpose staged through LDS so both
//               the read and the write are coalesced);
//   k_norm      s = 1 / (sqrt(sum of partials) + eps) per matrix, summed in a fixed order
//               (it also clears the contraction kernels' tail-split counters; the step's
//               first momentum launch clears them and the workspace's status word too);
//   k_adamw     AdamW on the packed fp32 tail.
// Method: DMuon summary §1 (Newton-Schulz on momentum-aggregated gradients); MatrixFSDP
// summary, Methodology §1 (AdamW for the non-matrix tail).
#include <hip/hip_runtime.h>

#include "muon_internal.h"

using namespace muon;

namespace {

__device__ __forceinline__ float ld_f(const uint16_t* p) {
  return __uint_as_float(uint32_t(*p) << 16);
}
__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float as_f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ float as_f(float f) { return f; }

// Round to the storage type (round to nearest even for bf16).
__device__ __forceinline__ void st_f(uint16_t* p, float f) {
  *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ void st_f(float* p, float f) { *p = f; }
__device__ __forceinline__ float round_to(float f, const uint16_t*) {
  return as_f(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}
__device__ __forceinline__ float round_to(float f, const float*) { return f; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 16-byte chunk of S elements.
template <typename S>
struct Chunk {
  static constexpr int N = 16 / sizeof(S);
  S v[N];
};

// 16-byte global accesses through address-space-1 pointers: the buffer pointers come from
// the descriptor table (generic), and FLAT accesses would also hold up the LDS waits.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4* g_u32x4;
typedef __attribute__((address_space(1))) const u32x4* g_cu32x4;

template <typename S>
__device__ __forceinline__ void load_chunk(const S* p, Chunk<S>& c) {
  *reinterpret_cast<u32x4*>(c.v) = *(g_cu32x4)(p);
}
template <typename S>
__device__ __forceinline__ void store_chunk(S* p, const Chunk<S>& c) {
  *(g_u32x4)(p) = *reinterpret_cast<const u32x4*>(c.v);
}

// A chunk's values widened to fp32 (8 bf16 -> two 16-byte stores); p is 16-byte aligned.
template <typename S>
__device__ __forceinline__ void store_f32(float* p, const Chunk<S>& c) {
  float f[Chunk<S>::N];
#pragma unroll
  for (int e = 0; e < Chunk<S>::N; ++e) f[e] = as_f(c.v[e]);
#pragma unroll
  for (int q = 0; q < Chunk<S>::N / 4; ++q) *(g_u32x4)(p + 4 * q) = *reinterpret_cast<const u32x4*>(f + 4 * q);
}

template <typename S>
__global__ __launch_bounds__(256) void k_momentum(MomArgs a) {
  constexpr int CH = 16 / sizeof(S);  // elements per 16-byte chunk
  constexpr int CPR = kEwTile / CH;   // chunks per tile row
  constexpr int RPP = 256 / CPR;      // tile rows per pass
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float red[4];

  if (a.status && blockIdx.x == 0) {
    if (threadIdx.x == 0) *a.status = 0;
    for (int i = threadIdx.x; i < a.split_cnt_n; i += 256) a.split_cnt[i] = 0;
  }
  const int vt = a.tile_begin + int(blockIdx.x);
  int lo = a.first, hi = a.last - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.desc[mid].mom_prefix <= vt) lo = mid; else hi = mid - 1;
  }
  const MatDesc& d = a.desc[lo];
  const int t = vt - d.mom_prefix;
  const int i0 = (t / d.mom_tiles_c) * kEwTile;
  const int j0 = (t % d.mom_tiles_c) * kEwTile;
  const int r = d.rows, c = d.cols;
  const S* G = static_cast<const S*>(d.grad);
  S* M = static_cast<S*>(d.mom);
  S* copy = static_cast<S*>(d.copy_out);
  const float beta = a.beta;
  const int tid = threadIdx.x;
  const int lr = tid / CPR;
  const int lc = (tid % CPR) * CH;
  float ss = 0.0f;

#pragma unroll
  for (int pass = 0; pass < kEwTile / RPP; ++pass) {
    const int li = pass * RPP + lr;
    const int gi = i0 + li;
    const int gj = j0 + lc;
    Chunk<S> out;
    if (gi < r) {
      const int64_t base = int64_t(gi) * c + gj;
      if (!M) {  // no momentum buffer: M' = G, only the copies and sums are written
        if (d.vec && gj + CH <= c) {
          load_chunk(G + base, out);
        } else {
#pragma unroll
          for (int e = 0; e < CH; ++e) {
            if (gj + e < c) out.v[e] = G[base + e];
            else st_f(&out.v[e], 0.0f);
          }
        }
      } else if (d.vec && gj + CH <= c) {
        Chunk<S> gv, mv;
        load_chunk(G + base, gv);
        load_chunk(M + base, mv);
#pragma unroll
        for (int e = 0; e < CH; ++e) st_f(&out.v[e], fmaf(beta, as_f(mv.v[e]), as_f(gv.v[e])));
        store_chunk(M + base, out);
      } else {
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          if (gj + e < c) {
            st_f(&out.v[e], fmaf(beta, ld_f(M + base + e), ld_f(G + base + e)));
            M[base + e] = out.v[e];
          } else {
            st_f(&out.v[e], 0.0f);
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < CH; ++e) st_f(&out.v[e], 0.0f);
    }
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const float x = as_f(out.v[e]);
      ss = fmaf(x, x, ss);
      tile[li][lc + e] = x;
    }
    // Same-orientation zero-padded copy: rows < r, columns < round_up(c, 64); fp32 for a bf16
    // matrix whose Gram iteration runs in fp32.
    if (copy && gi < r) {
      if (sizeof(S) == 2 && d.gram_f32) store_f32(static_cast<float*>(d.copy_out) + int64_t(gi) * d.copy_ld + gj, out);
      else store_chunk(copy + int64_t(gi) * d.copy_ld + gj, out);
    }
  }

  // Transposed copy: row j (< c) holds column j of M'; columns < round_up(r, 64).
  S* trans = static_cast<S*>(d.trans_out);
  if (trans) {
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < kEwTile / RPP; ++pass) {
      const int lj = pass * RPP + lr;
      const int gj = j0 + lj;
      if (gj < c) {
        Chunk<S> o;
#pragma unroll
        for (int e = 0; e < CH; ++e) st_f(&o.v[e], tile[lc + e][lj]);
        if (sizeof(S) == 2 && d.gram_f32)
          store_f32(static_cast<float*>(d.trans_out) + int64_t(gj) * d.trans_ld + i0 + lc, o);
        else
          store_chunk(trans + int64_t(gj) * d.trans_ld + i0 + lc, o);
      }
    }
  }

  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) a.partials[vt] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_norm(NormArgs a) {
  __shared__ double red[256];
  const MatDesc& d = a.desc[blockIdx.x];
  const int ntiles = d.mom_tiles_r * d.mom_tiles_c;
  double acc = 0.0;
  for (int t = threadIdx.x; t < ntiles; t += 256) acc += double(a.partials[d.mom_prefix + t]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.scale[blockIdx.x] = float(1.0 / (sqrt(red[0]) + double(a.eps)));
  // The contractions' tail-split counters start every step at zero (each tile's last piece
  // clears its own pair again when it is done).
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.split_cnt_n; i += 256) a.split_cnt[i] = 0;
}

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const AdamArgs& a) {
  m = fmaf(a.beta1, m, (1.0f - a.beta1) * g);
  v = fmaf(a.beta2, v, (1.0f - a.beta2) * g * g);
  const float mh = m / a.bc1;
  const float vh = v / a.bc2;
  p = p - a.lr * (mh / (sqrtf(vh) + a.eps) + a.wd * p);
}

__global__ __launch_bounds__(256) void k_adamw(AdamArgs a) {
  const int64_t stride = int64_t(gridDim.x) * 256 * 4;
  const bool vec = ((reinterpret_cast<uintptr_t>(a.p) | reinterpret_cast<uintptr_t>(a.g) |
                     reinterpret_cast<uintptr_t>(a.m) | reinterpret_cast<uintptr_t>(a.v)) & 15) == 0;
  for (int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4; i < a.n; i += stride) {
    if (vec && i + 4 <= a.n) {
      float4 p = *reinterpret_cast<const float4*>(a.p + i);
      const float4 g = *reinterpret_cast<const float4*>(a.g + i);
      float4 m = *reinterpret_cast<const float4*>(a.m + i);
      float4 v = *reinterpret_cast<const float4*>(a.v + i);
      adamw_one(p.x, g.x, m.x, v.x, a);
      adamw_one(p.y, g.y, m.y, v.y, a);
      adamw_one(p.z, g.z, m.z, v.z, a);
      adamw_one(p.w, g.w, m.w, v.w, a);
      *reinterpret_cast<float4*>(a.p + i) = p;
      *reinterpret_cast<float4*>(a.m + i) = m;
      *reinterpret_cast<float4*>(a.v + i) = v;
    } else {
      for (int64_t j = i; j < i + 4 && j < a.n; ++j) {
        float p = a.p[j], m = a.m[j], v = a.v[j];
        adamw_one(p, a.g[j], m, v, a);
        a.p[j] = p;
        a.m[j] = m;
        a.v[j] = v;
      }
    }
  }
}

}  // namespace

int muon_launch_momentum(const MomArgs& a, int dtype, void* stream) {
  if (a.total_tiles <= 0) return hipSuccess;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_momentum<uint16_t>, dim3(a.total_tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_momentum<float>, dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

int muon_launch_norm(const NormArgs& a, void* stream) {
  if (a.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_norm, dim3(a.count), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError();
}

int muon_launch_adamw(const AdamArgs& a, void* stream) {
  if (a.n <= 0) return hipSuccess;
  const int64_t per_block = 256 * 4;
  int64_t blocks = (a.n + per_block - 1) / per_block;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(k_adamw, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError();
}
