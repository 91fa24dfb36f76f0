// Quantize-append kernel: TurboQuant encode of new K/V rows into the packed
// cache ("TurboQuant KV Cache Quantization in MLX-VLM": "The TurboQuantKVCache
// Class", "Fused vs. Separate Quantization Paths"; mlxcel "TurboQuant KV
// cache": "Available modes" for the fp16 and delegated sides).
//
// One launch handles both sides.  A group of D/4 lanes owns one row (four
// consecutive fp16 elements per lane): it reduces the squared norm across
// the group, applies the sign diagonal and the Walsh-Hadamard butterflies
// (two strides inside the lane, the rest across lanes with shuffles), scales
// by 1/(n sqrt(D)), finds each code by binary search over the thresholds and
// assembles the LSB-first words with shuffles, so each packed row leaves in
// one coalesced store.
#include <stdlib.h>
#include <string.h>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kBlock = 256;

// TQ_QUANTIZE_VARIANT=plain forces the kernel below for every side (A/B
// measurements and the cross-check tests).
bool getenv_plain() {
  const char *e = getenv("TQ_QUANTIZE_VARIANT");
  return e && strcmp(e, "plain") == 0;
}

// Encode one row held as four elements per lane.  Writes words and norm when
// `write` is set for this group (all lanes of the wave must call this, since
// it shuffles).
template <int D>
__device__ __forceinline__ void encode_row(const float (&x)[4], int t,
                                           const uint32_t *sign, const float *thr,
                                           int bits, int words, bool write,
                                           uint32_t *row_out, float *norm_out) {
  constexpr int TPR = D / 4;
  float v[4];
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += x[e] * x[e];
  ss = group_sum<TPR>(ss);
  const float n = sqrtf(ss);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = x[e] * sign_of(sign, 4 * t + e);
  fwht_group4<TPR>(v, t);
  const float inv = (n > 0.0f) ? 1.0f / (n * sqrtf(static_cast<float>(D))) : 0.0f;
  uint32_t chunk = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = count_below(thr, bits, v[e] * inv);
    chunk |= static_cast<uint32_t>(c) << (bits * e);
  }
  // Word w gathers the 4*bits-bit chunks of lanes t0 .. t0 + kmax - 1.
  const int cb = 4 * bits;
  const int kmax = (32 + cb - 1) / cb + 1;
  const int w = t;
  const int t0 = (32 * w) / cb;
  uint32_t word = 0;
  for (int k = 0; k < kmax; ++k) {
    const int src = t0 + k;
    const uint32_t c = __shfl(chunk, src < TPR ? src : TPR - 1, TPR);
    const int sh = cb * src - 32 * w;
    if (src < TPR && sh < 32 && sh > -cb) word |= (sh >= 0) ? (c << sh) : (c >> (-sh));
  }
  if (write) {
    if (w < words) row_out[w] = word;
    if (t == 0) *norm_out = n;
  }
}

// INT8 per-token absmax (mlxcel "TurboQuant KV cache", "Available modes"):
// a = max|x|, code = 127 x / a rounded to the nearest integer (ties to even),
// taken exactly; the stored scale is a / 127 in float32.  127 x is exact in
// float32 (an fp16 significand times 7 bits), so the correctly rounded
// quotient is within one code of the answer, and the sign of 2 (127 x) -
// (2 k +- 1) a, computed by one fma (an exact product, one rounding, which
// keeps the sign and zero), says on which side of k +- 1/2 the exact
// quotient lies.  Lane t writes word t of the row (its four codes,
// coordinate 4 t + e in byte e).
template <int D>
__device__ __forceinline__ void encode_int8(const float (&x)[4], int t, bool write, uint32_t *row_out,
                                            float *scale_out) {
  constexpr int TPR = D / 4;
  float a = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  a = group_max<TPR>(a);
  const float scale = a / 127.0f;
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = a > 0.0f ? int8_code(x[e], a) : 0;
    w |= (static_cast<uint32_t>(c) & 0xffu) << (8 * e);
  }
  if (write) {
    row_out[t] = w;
    if (t == 0) *scale_out = scale;
  }
}

template <int D>
__device__ __forceinline__ void load4(const uint16_t *src, int t, float (&x)[4]) {
  const uint2 raw = *reinterpret_cast<const uint2 *>(src + 4 * t);
  x[0] = h2f(static_cast<uint16_t>(raw.x & 0xffffu));
  x[1] = h2f(static_cast<uint16_t>(raw.x >> 16));
  x[2] = h2f(static_cast<uint16_t>(raw.y & 0xffffu));
  x[3] = h2f(static_cast<uint16_t>(raw.y >> 16));
}

__device__ __forceinline__ void copy4(const uint16_t *src, uint16_t *dst, int t) {
  *reinterpret_cast<uint2 *>(dst + 4 * t) = *reinterpret_cast<const uint2 *>(src + 4 * t);
}

template <int D>
__global__ __launch_bounds__(kBlock) void quantize_append_kernel(const QuantizeParams p) {
  constexpr int TPR = D / 4;
  __shared__ float thr[2][kMaxLevels];
  for (int i = threadIdx.x; i < kMaxLevels; i += kBlock) {
    thr[0][i] = p.k_thr[i];
    thr[1][i] = p.v_thr[i];
  }
  __syncthreads();

  const int t = threadIdx.x % TPR;
  const long per_side = static_cast<long>(p.batch) * p.heads * p.n_new;
  // tasks: rows of the sides in p.side_mask (K rows first)
  const long first = (p.side_mask == 2) ? per_side : 0;
  const long n_tasks = (p.side_mask == 3) ? 2 * per_side : per_side;
  const long task = first + static_cast<long>(blockIdx.x) * (kBlock / TPR) + threadIdx.x / TPR;
  // Out-of-range groups still run the shuffles of a (dummy) row so that the
  // wave stays converged; they store nothing.
  const bool live = task < first + n_tasks;
  const int side = live ? static_cast<int>(task / per_side) : 0;
  const long r = live ? task % per_side : 0;
  const long bh = r / p.n_new;
  const int i = static_cast<int>(r % p.n_new);
  const int pos = p.offset + i;
  const SideDev &s = side ? p.v : p.k;
  const uint16_t *src = (side ? p.v_new : p.k_new) + (bh * p.n_new + i) * D;
  const float *th = thr[side];
  // the storage row; a position in a block outside the paged pools is not
  // written (-1)
  const long srow = cache_row(p.pg, bh, pos, p.capacity);
  const bool put = live && srow >= 0;
  const long orow = srow < 0 ? 0L : srow;

  if (s.mode == TQ_SIDE_INT8) {
    float x[4];
    load4<D>(src, t, x);
    encode_int8<D>(x, t, put, s.codes + orow * s.words, s.norms + orow);
  } else if (s.mode == TQ_SIDE_PACKED) {
    float x[4];
    load4<D>(src, t, x);
    encode_row<D>(x, t, p.sign, th, s.bits, s.words, put, s.codes + orow * s.words, s.norms + orow);
  } else if (s.mode == TQ_SIDE_FP16) {
    if (put) copy4(src, s.fp16 + orow * D, t);
  } else {  // TQ_SIDE_DELEGATED (V only)
    const int hot = s.hot;
    const int end = p.offset + p.n_new;
    if (pos < end - hot) {
      // Already older than the newest `hot` positions: straight to cold.
      float x[4];
      load4<D>(src, t, x);
      encode_row<D>(x, t, p.sign, th, s.bits, s.words, put, s.codes + orow * s.words, s.norms + orow);
    } else {
      // Last new position of its ring slot: evict the slot's old occupant
      // (the position o < offset with o = pos mod hot) into the cold rows,
      // then overwrite the slot.  No other group touches this slot.
      const int slot = pos % hot;
      const int o = pos - hot * ((pos - p.offset) / hot + 1);
      uint16_t *ring = s.fp16 + (bh * hot + slot) * D;
      float x[4];
      load4<D>(ring, t, x);
      const long erow = cache_row(p.pg, bh, o >= 0 ? o : 0, p.capacity);
      encode_row<D>(x, t, p.sign, th, s.bits, s.words, live && o >= 0 && erow >= 0,
                    s.codes + (erow < 0 ? 0L : erow) * s.words, s.norms + (erow < 0 ? 0L : erow));
      if (live) copy4(src, ring, t);
    }
  }
}

template <int D>
hipError_t launch_d(const QuantizeParams &p, hipStream_t stream) {
  constexpr int TPR = D / 4;
  const long tasks = (p.side_mask == 3 ? 2L : 1L) * p.batch * p.heads * p.n_new;
  const long blocks = (tasks + (kBlock / TPR) - 1) / (kBlock / TPR);
  hipLaunchKernelGGL(quantize_append_kernel<D>, dim3(static_cast<unsigned>(blocks)),
                     dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Packed sides at head_dim 128 with 1..4 bits and appends of at least 16
// rows go to the matrix-core encoder; everything else (other head sizes and
// widths, fp16 copies, the delegated ring, short appends) to the kernel
// above.  Both write the same bytes.
hipError_t launch_quantize_append(const QuantizeParams &p, hipStream_t stream) {
  QuantizeParams m = p;
  m.k_lut_scale = m.v_lut_scale = 0.0f;
  int rest = 3;
  if (p.head_dim == 128 && p.n_new >= 16 && !getenv_plain()) {
    for (int side = 0; side < 2; ++side) {
      const SideDev &s = side ? p.v : p.k;
      if (s.mode != TQ_SIDE_PACKED || s.bits < 1 || s.bits > 4) continue;
      const float sc = quantize_lut_scale(side ? p.v_thr : p.k_thr, s.bits);
      if (sc <= 0.0f) continue;
      (side ? m.v_lut_scale : m.k_lut_scale) = sc;
      rest &= ~(1 << side);
    }
  }
  if (rest != 3) {
    const hipError_t e = launch_quantize_mfma(m, stream);
    if (e != hipSuccess) return e;
  }
  if (rest == 0) return hipSuccess;
  QuantizeParams q = p;
  q.side_mask = rest;
  switch (p.head_dim) {
    case 32: return launch_d<32>(q, stream);
    case 64: return launch_d<64>(q, stream);
    case 128: return launch_d<128>(q, stream);
    case 256: return launch_d<256>(q, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
