// Completion of a tile whose contraction the tail split (tile_order.h) cut into pieces run
// by different workgroups.  Shared by both MFMA kernels; device code only.
//
// The counter protocol (arrive, publish, collect, and what a timeout leaves behind) is in
// split_protocol.h, shared with a host emulation.  Here: every piece but the last stores its
// fp32 partial sums in its own slot before publishing; the last piece adds the others' sums
// to its own in piece order and goes on to the tile's epilogue, or, if its bounded wait ran
// out, stores NaN for the whole tile.  Adding in piece order makes the result independent
// of which piece finishes last: each element is ((p0 + p1) + p2) + ..., the own piece taken
// from registers at its place.
//
// Coherence.  The pieces of a tile may run on different XCDs, whose L2 caches are not
// coherent with each other.  Every access to a slot and to the counters is made at device
// scope (the sc1 cache policy: device-scope stores are complete only once visible to every
// XCD, device-scope loads do not return a stale line), so neither side needs a device-wide
// fence, which would write back or invalidate the whole L2 of its XCD under the other
// workgroups' feet.  A writer's stores are complete (s_waitcnt) before its count is made;
// the reader issues its loads only after it has seen the count.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "split_protocol.h"

namespace muon {

// Device-scope atomics of the protocol (the pieces of a tile may run on different XCDs).
struct DeviceSplitOps {
  __device__ int32_t fetch_add(int32_t* p, int32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ int32_t load(int32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
  __device__ void store(int32_t* p, int32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
  __device__ void pause() { __builtin_amdgcn_s_sleep(8); }
};

// Accumulator layout shared by writer and reader (both run the same kernel and tile shape):
// float4 number ((wave * FM + i) * FN + j) * 4 + r4 of a slot holds lane-interleaved values
// acc[i][j][4 r4 .. 4 r4 + 3] of that wave, 64 lanes apart, so each store and load
// instruction covers 1 KB of consecutive bytes.
constexpr int kCpolDevice = 16;  // cache policy operand of the buffer builtins: sc1 (device scope)

typedef unsigned int split_u32x4 __attribute__((ext_vector_type(4)));

template <int FM, int FN, typename Acc>
__device__ __forceinline__ bool split_fixup(Acc (&acc)[FM][FN], int piece, int pieces, int32_t* cnt,
                                            float* slots, int64_t slot_floats, int* flag, bool idle,
                                            int32_t* status, int spin_limit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  DeviceSplitOps ops;
  // flag[0]: the count this piece saw on arrival (kept as the count: reading a 0/1 flag here
  // instead made the compiler spill inside both kernels' main loops); flag[1]: 0 once the
  // last piece's wait has seen the others' sums, 1 if it timed out.
  if (tid == 0) flag[0] = split_arrive_count(ops, cnt);
  __syncthreads();
  const bool last = split_is_last(flag[0], pieces);
  // The tile's slots as one buffer (at most kMaxPieces x 384 KB); byte offset of float4 q of
  // slot p: (p slot_floats + 4 q) 4.
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(slots, (short)0, int(int64_t(pieces) * slot_floats * 4), 0x00020000);
  const uint32_t base = uint32_t(wave * FM * FN * 4 * 64 + lane) * 16u;
  auto at = [&](int p, int i, int j, int r4) -> uint32_t {
    return uint32_t(p) * uint32_t(slot_floats * 4) + base + uint32_t((i * FN + j) * 4 + r4) * 1024u;
  };
  if (!last) {
    if (!idle) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 v = make_float4(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                                         acc[i][j][4 * r4 + 3]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(split_u32x4, v), rsrc, at(piece, i, j, r4),
                                                   0, kCpolDevice);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete (visible to every XCD)
    __syncthreads();
    if (tid == 0) split_publish(ops, cnt);
    return false;
  }
  if (tid == 0) flag[1] = split_collect(ops, cnt, pieces, spin_limit, status) ? 0 : 1;
  __syncthreads();  // the slot loads below are issued after the count was seen
  // Timed out: every partial sum read below is taken as NaN (the loads still stay inside the
  // slots), so the tile is stored as NaN, and the status word says why.
  const bool ok = flag[1] == 0;
  auto load = [&](int p, int i, int j, int r4) -> float4 {
    const float4 x =
        __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, at(p, i, j, r4), 0, kCpolDevice));
    const float q = __builtin_nanf("");
    return ok ? x : make_float4(q, q, q, q);
  };
  if (!idle) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          // sum = ((p0 + p1) + ...) + p_last; the own piece enters at its place.
          float s0, s1, s2, s3;
          if (piece == 0) {
            s0 = acc[i][j][4 * r4];
            s1 = acc[i][j][4 * r4 + 1];
            s2 = acc[i][j][4 * r4 + 2];
            s3 = acc[i][j][4 * r4 + 3];
          } else {
            const float4 x = load(0, i, j, r4);
            s0 = x.x, s1 = x.y, s2 = x.z, s3 = x.w;
            for (int p = 1; p < piece; ++p) {
              const float4 y = load(p, i, j, r4);
              s0 += y.x, s1 += y.y, s2 += y.z, s3 += y.w;
            }
            s0 += acc[i][j][4 * r4];
            s1 += acc[i][j][4 * r4 + 1];
            s2 += acc[i][j][4 * r4 + 2];
            s3 += acc[i][j][4 * r4 + 3];
          }
          for (int p = piece + 1; p < pieces; ++p) {
            const float4 y = load(p, i, j, r4);
            s0 += y.x, s1 += y.y, s2 += y.z, s3 += y.w;
          }
          acc[i][j][4 * r4] = s0;
          acc[i][j][4 * r4 + 1] = s1;
          acc[i][j][4 * r4 + 2] = s2;
          acc[i][j][4 * r4 + 3] = s3;
        }
  }
  return true;
}

}  // namespace muon
