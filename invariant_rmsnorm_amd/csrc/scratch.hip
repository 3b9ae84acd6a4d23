// Library-held device scratch for rmsnorm_bwd_noalloc: the dgamma chunk
// partials of callers that cannot allocate device memory (code under graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope device array; each GPU the library runs on holds
// its own copy, at its own address, until the process ends. In host code the
// array's name is only a stand-in for the symbol, not a device address, so
// the host never passes it anywhere: scratch_ptr() asks the runtime for the
// address on the current device (hipGetSymbolAddress), once per device, and
// every use goes through that pointer.
#include <hip/hip_runtime.h>

#include <atomic>

#include "scratch.hpp"

static __device__ __align__(256) unsigned char scratch[rmsn::kScratchBytes];

namespace rmsn {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with `dev` current: the address of this device's copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return 0;
}

}  // namespace rmsn
