// Device scratch for the allocation-free entry point (muon_step_noalloc): a
// file-scope array in device memory that stands in for the caller-owned
// workspace. Each GPU the library runs on holds its own copy, at its own
// address, from the first use on that device until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace muon {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 256;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace muon
