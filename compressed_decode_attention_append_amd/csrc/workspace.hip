// Workspace set-up behind tq_decode_workspace_init: the decode's per-unit
// arrival counters (the workspace's first kCounterBytes) must read zero
// before a workspace's first use, and every successful decode leaves them
// zero.  A plain store kernel clears them (not a memset: a caller may record
// this into a HIP graph).
#include "tq_common.h"

namespace tq {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFillThreads = 256;

__global__ __launch_bounds__(kFillThreads) void zero_fill_kernel(u32x4_t *p, size_t n16) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kFillThreads + threadIdx.x;
  if (i < n16) p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_zero_fill(void *buf, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = (n16 + kFillThreads - 1) / kFillThreads;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kFillThreads), 0, stream,
                     static_cast<u32x4_t *>(buf), n16);
  return hipGetLastError();
}

}  // namespace tq
