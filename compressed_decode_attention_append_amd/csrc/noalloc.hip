// Fixed device scratch behind tq_decode_attention_noalloc, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops).  The decode's workspace (arrival counters, then the split
// partials) lives in one static device array per GPU instead of a caller's
// buffer.  Its host-side name is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever handed to a kernel.
#include <mutex>

#include "tq_common.h"

namespace tq {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on device i, once set up

}  // namespace

// The scratch of the device `stream` runs on: its device address, taken on
// the first call for that device (with the device made current for the
// lookup), when its counter region is also cleared on `stream`.
hipError_t scratch_workspace(hipStream_t stream, void **ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the counters must start at zero (each decode leaves them zero)
    e = launch_zero_fill(p, kCounterBytes, stream);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
