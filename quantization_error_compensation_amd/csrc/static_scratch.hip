// The library's own scratch memory, for callers that cannot allocate
// (spear_ec_linear_static): a file-scope device array of kStaticScratchBytes
// on every device the library runs on, held until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device (with that device current) and kept
// per device; only that address is handed to kernels.  Every call on a
// device shares its array, so calls that overlap on one device race, like
// calls that share one caller workspace.
#include <mutex>

#include "internal.hpp"

namespace spear {
namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The counter words at the head of a workspace start at zero (every call
// leaves them so): cleared once, when a device's array is first used.
__global__ __launch_bounds__(256) void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t static_scratch(void** out, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_words, dim3((kCounterSlots + 255) / 256), dim3(256), 0, st,
                       static_cast<uint32_t*>(p), kCounterSlots);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace spear
