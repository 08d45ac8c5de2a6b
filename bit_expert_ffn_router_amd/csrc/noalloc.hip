// The static device scratch behind moe_layer_forward_noalloc: the decode
// path's workspace (the routing, the list of selected experts and their h
// rows) for callers that cannot allocate device memory.  One copy of the
// array per GPU, held until the process ends; every call on a GPU shares it,
// so calls that overlap in time on one GPU race and must be ordered by the
// caller.  Nothing in it has to start at zero: each call writes every entry
// it later reads.
#include <atomic>
#include <mutex>

#include "kernels.hpp"

// In host code this name is only a stand-in for the symbol; the device
// address comes from hipGetSymbolAddress below, once per device.
static __device__ __align__(256) uint8_t scratch[moe::kNoAllocScratchBytes];

namespace moe {

hipError_t noalloc_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      // the device is current here: this is its copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace moe
