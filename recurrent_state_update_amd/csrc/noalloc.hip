// Static scratch for the prefill entry point that allocates nothing, gfx950.
//
// Callers that cannot allocate device memory (code under HIP graph capture, serving loops that
// forbid it) take their prefill scratch from one file-scope device array of kNoAllocScratchBytes
// instead of a workspace argument.  Each GPU the library runs on holds its own copy of the array
// from module load until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is a stand-in, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace m2 {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidValue;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace m2
