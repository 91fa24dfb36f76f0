// Streaming-read probe behind tq_read_probe: a measurement aid for the HBM
// read bandwidth a plain kernel attains, not part of the method.  One block
// of 768 threads per compute unit; each block reads a contiguous slice with
// 16-byte loads, two in flight per thread.  The sink receives the xor of all
// 32-bit words of the buffer (one atomic xor per wave), so no load can be
// dropped and the result is checkable.
#include "tq_common.h"

namespace tq {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 768;
constexpr int kProbeBlocks = 256;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t *__restrict__ p, size_t n16,
                                                                   unsigned *sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = static_cast<size_t>(blockIdx.x) * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (size_t i = lo + threadIdx.x; i < hi; i += 2 * static_cast<size_t>(kProbeThreads)) {
    const size_t j = i + kProbeThreads;
    const u32x4_t a = __builtin_nontemporal_load(p + i);
    const u32x4_t b = j < hi ? __builtin_nontemporal_load(p + j) : u32x4_t{0u, 0u, 0u, 0u};
    acc ^= a ^ b;
  }
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

__global__ void zero_kernel(unsigned *sink) {
  if (threadIdx.x == 0) atomicExch(sink, 0u);
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, unsigned *sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, stream, sink);
  if (n16 > 0) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4_t *>(buf), n16, sink);
  }
  return hipGetLastError();
}

}  // namespace tq
