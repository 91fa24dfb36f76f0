// Device helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// 512 zero bytes (the longest stored row: fp16 at head_dim 256).  A position
// in a block outside the paged pools reads its row from here.  Global memory
// on purpose, not const: a const array lands in the constant address space,
// and a pointer that may point there or into the cache turns the kernels'
// row loads into flat loads, which the LDS waits then also wait for.  Never
// written.
static __device__ uint32_t kZeroRow[128] = {};

__device__ __forceinline__ float h2f(uint16_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

__device__ __forceinline__ uint16_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Sign s_j of the rotation (+1 / -1) from the packed sign words.
__device__ __forceinline__ float sign_of(const uint32_t *sign, int j) {
  return ((sign[j >> 5] >> (j & 31)) & 1u) ? -1.0f : 1.0f;
}

// Walsh-Hadamard butterflies over one row held by a group of TPR lanes, four
// consecutive elements per lane (lane t of the group holds elements
// 4t .. 4t+3).  Strides 1 and 2 are inside the lane, strides 4, 8, ... pair
// lane t with lane t ^ (stride / 4).  Butterfly (a, b) -> (a + b, a - b),
// strides in increasing order: the natural-order Sylvester transform.
template <int TPR>
__device__ __forceinline__ void fwht_group4(float (&v)[4], int t) {
  const float a0 = v[0] + v[1], a1 = v[0] - v[1];
  const float a2 = v[2] + v[3], a3 = v[2] - v[3];
  v[0] = a0 + a2;
  v[2] = a0 - a2;
  v[1] = a1 + a3;
  v[3] = a1 - a3;
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) {
    const bool upper = (t & m) != 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o = __shfl_xor(v[e], m);
      v[e] = upper ? (o - v[e]) : (v[e] + o);
    }
  }
}

// Sum over the TPR lanes of a group (all lanes receive the total).
template <int TPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Maximum over the TPR lanes of a group (all lanes receive it).
template <int TPR>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Signed byte j % 4 of word w, as a float (INT8 rows: coordinate j in byte j).
__device__ __forceinline__ float int8_at(uint32_t w, int j) {
  return static_cast<float>(static_cast<int8_t>((w >> (8 * (j & 3))) & 0xffu));
}

// Number of thresholds strictly below y: branch-free binary search over the
// ascending array thr[0 .. 2^bits - 2].
__device__ __forceinline__ int count_below(const float *thr, int bits, float y) {
  int code = 0;
  for (int s = bits - 1; s >= 0; --s) {
    const int cand = code + (1 << s);
    code = (y > thr[cand - 1]) ? cand : code;
  }
  return code;
}

// INT8 absmax code of x in a row whose largest magnitude is a > 0:
// round(127 x / a) to nearest, ties to even, decided exactly.  2 (127 x) =
// 254 x is exact in float; a first guess k from the rounded division is
// moved by one where the exact signs of 127 x / a - (k +- 1/2), taken by
// fused multiply-adds, say it lies past a half step.
__device__ __forceinline__ int int8_code(float x, float a) {
  const float y2 = 254.0f * x;  // 2 (127 x), exact
  float k = rintf(0.5f * y2 / a);
  const float up = fmaf(-(2.0f * k + 1.0f), a, y2);  // sign of 127 x / a - (k + 1/2)
  const float dn = fmaf(-(2.0f * k - 1.0f), a, y2);  // sign of 127 x / a - (k - 1/2)
  const bool odd = (static_cast<int>(k) & 1) != 0;
  if (up > 0.0f || (up == 0.0f && odd)) {
    k += 1.0f;
  } else if (dn < 0.0f || (dn == 0.0f && odd)) {
    k -= 1.0f;
  }
  return min(127, max(-127, static_cast<int>(k)));
}

// Extract code j (bits wide) from a packed LSB-first row.
__device__ __forceinline__ uint32_t extract_code(const uint32_t *row, int bits, int j) {
  const int o = bits * j;
  const int w = o >> 5;
  const int sh = o & 31;
  uint32_t v = row[w] >> sh;
  if (sh + bits > 32) v |= row[w + 1] << (32 - sh);
  return v & ((1u << bits) - 1u);
}

}  // namespace tq
