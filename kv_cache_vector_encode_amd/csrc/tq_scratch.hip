// tq_scratch: the fixed device buffer of tq_decode_attend_noalloc, for
// callers that cannot allocate device memory (code under graph capture,
// serving loops that forbid allocation).  It holds the decode's per-split
// partial results instead of a caller workspace.
//
// The array lives in the library's code object, one copy per GPU the library
// runs on, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in symbol): the first call
// on each device, with that device current, resolves the device's own copy
// with hipGetSymbolAddress and keeps that address for the device.

#include <hip/hip_runtime.h>

#include <mutex>

#include "tq_internal.h"

namespace tq {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

int scratch_buffer(void** ptr, int64_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  *bytes = kScratchBytes;
  return 0;
}

}  // namespace tq
