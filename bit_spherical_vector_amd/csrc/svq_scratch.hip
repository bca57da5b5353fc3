// Library-held scratch for svq_linear_noalloc, the entry point for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc).
//
// The array lives in the code object: each GPU the library runs on holds its
// own copy, allocated when the module is loaded and kept until the process
// ends.  Host code never passes the array's name to a kernel (in host code it
// is only a stand-in for the symbol); the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and is cached per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "svq_internal.h"

static __device__ __align__(256) uint8_t scratch[svq::SCRATCH_BYTES];

namespace svq {

hipError_t scratch_ptr(void **ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void *cached[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    cached[dev] = p;
  }
  *ptr = cached[dev];
  return hipSuccess;
}

}  // namespace svq
