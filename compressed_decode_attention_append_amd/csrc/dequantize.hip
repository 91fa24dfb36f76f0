// Dequantize packed rows back to fp32: x~ = n diag(s) H c[code] / sqrt(d)
// ("TurboQuant KV Cache Quantization in MLX-VLM", FAQ "Where is the
// dequantization logic implemented?": the stored rotation and codebooks turn
// the packed words back into float32).  A check path, not on the decode.
//
// A group of D/4 lanes owns one row, four consecutive coordinates per lane,
// and applies the same butterflies as the encoder (H is symmetric).
#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kBlock = 256;

template <int D>
__global__ __launch_bounds__(kBlock) void dequantize_kernel(const DequantParams p) {
  constexpr int TPR = D / 4;
  __shared__ float cent[kMaxLevels];
  for (int i = threadIdx.x; i < kMaxLevels; i += kBlock) cent[i] = p.cent[i];
  __syncthreads();
  const int t = threadIdx.x % TPR;
  const long rows = static_cast<long>(p.batch) * p.heads * p.count;
  const long task = static_cast<long>(blockIdx.x) * (kBlock / TPR) + threadIdx.x / TPR;
  const bool live = task < rows;
  const long r = live ? task : 0;
  const long bh = r / p.count;
  const int pos = p.start + static_cast<int>(r % p.count);
  // a position in a block outside the paged pools reads the zero row
  const long sr = cache_row(p.pg, bh, pos, p.capacity);
  const uint32_t *row = sr < 0 ? kZeroRow : p.s.codes + sr * p.s.words;
  const float n = sr < 0 ? 0.0f : p.s.norms[sr];
  if (p.s.mode == TQ_SIDE_INT8) {
    // INT8 rows: code times the row's scale, no rotation
    const uint32_t w = row[t];
    const float sc = n;
    if (live) {
      const float4 o = make_float4(int8_at(w, 0) * sc, int8_at(w, 1) * sc, int8_at(w, 2) * sc, int8_at(w, 3) * sc);
      *reinterpret_cast<float4 *>(p.out + r * D + 4 * t) = o;
    }
    return;
  }
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = cent[extract_code(row, p.s.bits, 4 * t + e)];
  fwht_group4<TPR>(v, t);
  const float scale = n / sqrtf(static_cast<float>(D));
  if (live) {
    float4 o;
    o.x = v[0] * sign_of(p.sign, 4 * t + 0) * scale;
    o.y = v[1] * sign_of(p.sign, 4 * t + 1) * scale;
    o.z = v[2] * sign_of(p.sign, 4 * t + 2) * scale;
    o.w = v[3] * sign_of(p.sign, 4 * t + 3) * scale;
    *reinterpret_cast<float4 *>(p.out + r * D + 4 * t) = o;
  }
}

template <int D>
hipError_t launch_d(const DequantParams &p, hipStream_t stream) {
  constexpr int TPR = D / 4;
  const long rows = static_cast<long>(p.batch) * p.heads * p.count;
  const long blocks = (rows + (kBlock / TPR) - 1) / (kBlock / TPR);
  hipLaunchKernelGGL(dequantize_kernel<D>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const DequantParams &p, hipStream_t stream) {
  switch (p.head_dim) {
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 256: return launch_d<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
