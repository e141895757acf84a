// Device scratch of mla_decode_paged_noalloc: the decode workspace (tile
// plan, partial outputs, partial lse) in a file-scope device array instead of
// caller memory, for callers that cannot allocate.  The array exists once per
// device the library is loaded on and lives until the process ends; every
// call on a device shares it.
#include <hip/hip_runtime.h>

#include <atomic>

#include "mla_internal.hpp"

static __device__ __align__(256) char scratch[mla::kNoAllocScratchBytes];

namespace mla {
namespace {

constexpr int kMaxDevices = 64;
// device address of `scratch` on each device, fetched once (a racing first
// call stores the same value)
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with this device current: its own copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace mla
