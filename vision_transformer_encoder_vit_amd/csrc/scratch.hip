// Device scratch owned by the library, for the forward entry point that
// allocates nothing (vit_block_forward_static): one file-scope array, which
// the runtime places on every GPU the library runs on, looked up once per
// device and kept until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace vit {

static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* per_device[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    // the array's device address on the current device (the name itself is
    // only a host-side stand-in)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace vit
