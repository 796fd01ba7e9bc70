// scratch.hip -- the fixed device buffer behind tq_decode_attend_noalloc.
//
// One array per GPU, in the library's code object, so callers that may not
// allocate (code under graph capture, serving loops, harnesses that forbid
// hipMalloc) still get the per-split partials the decode-attend kernels write.
// In host code `scratch` names a host-side stand-in, never the device memory:
// every host use goes through the address hipGetSymbolAddress returns, looked
// up once per device with that device current and kept here.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/tq.h"
#include "kernels.hpp"

namespace {

static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace tq {

hipError_t scratch_region(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255)) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
