// Device scratch of the allocation-free entry point (muon_step_noalloc), and a way to put a
// small host block into device memory with no host staging buffer: the block travels in the
// kernel arguments of a copy kernel.
//
// `scratch` is one file-scope device array per GPU, of kNoAllocBytes, held by every device
// the library's code object is loaded on until the process ends.  Host code never uses the
// array's name as an address (in host code it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, asked once per device with that device current,
// and is kept per device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "muon_internal.h"

namespace {

static __device__ __align__(256) char scratch[muon::kNoAllocBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device (nullptr: not asked yet)

// One kernel-argument block: n 32-bit words (at most kArgWords, 3 KB of data).
constexpr int kArgWords = 768;
struct ArgWords {
  uint32_t n;
  uint32_t w[kArgWords];
};

__global__ __launch_bounds__(256) void k_put_words(uint32_t* dst, ArgWords a) {
  for (uint32_t i = threadIdx.x; i < a.n; i += 256) dst[i] = a.w[i];
}

}  // namespace

int muon_noalloc_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return int(hipSuccess);
}

int muon_put_words(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0) return int(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* p = static_cast<const char*>(src);
  uint32_t* d = static_cast<uint32_t*>(dst);
  for (size_t done = 0; done < bytes;) {
    ArgWords a;
    const size_t words = std::min(size_t(kArgWords), (bytes - done) / 4);
    a.n = uint32_t(words);
    std::memcpy(a.w, p + done, words * 4);
    hipLaunchKernelGGL(k_put_words, dim3(1), dim3(256), 0, s, d + done / 4, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return int(e);
    done += words * 4;
  }
  return int(hipSuccess);
}
