// Decode attention straight from the packed cache: the plain split-context
// variant ("TurboQuant KV Cache Quantization in MLX-VLM", "How TurboQuant KV
// Cache Quantization Works": scores from the compressed representation; FAQ
// on dequantization: the stored rotation and codebooks).
//
// Grid (n_splits, B * Hkv); one block handles the G query heads of one KV
// head over one contiguous range of positions:
//   1. q is rotated once: R q = H diag(s) q / sqrt(d) by butterflies in LDS;
//      the softmax scale 1/sqrt(d) and log2(e) are folded in.
//   2. score of position i: n_i <R q, c[code_i]> (packed K) or q . k_i
//      (fp16 K), one thread per (position, head).
//   3. running max and sum per head (base-2 exponent).
//   4. value accumulation, one thread per (head, coordinate): packed rows
//      accumulate p_i n_i c[code_i,j] in the rotated domain; fp16 rows (fp16
//      V, or the delegated hot window) accumulate p_i v_ij as they are.
//   5. partial (max, sum, rotated sum, plain sum) to the workspace.
// A second kernel merges the splits by their maxima, applies the inverse
// rotation diag(s) H / sqrt(d) once per output head, adds the plain part and
// divides by the sum.
#include <math.h>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ float block_reduce(float x, float *red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(x, m);
    x = is_max ? fmaxf(x, o) : x + o;
  }
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kBlock / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// Is V row `t` served from fp16 storage?  Returns the fp16 row or null.
__device__ __forceinline__ const uint16_t *v_plain_row(const DecodeParams &p, long bk, int t) {
  const int D = p.head_dim;
  if (p.v.mode == TQ_SIDE_FP16) return p.v.fp16 + cache_row(p.pg, bk, t, p.capacity) * D;
  if (p.v.mode == TQ_SIDE_DELEGATED && t >= p.length - p.v.hot)
    return p.v.fp16 + (bk * p.v.hot + (t % p.v.hot)) * D;
  return nullptr;
}

template <int D>
__global__ __launch_bounds__(kBlock) void decode_split_kernel(const DecodeParams p) {
  extern __shared__ float smem[];
  const int G = p.q_heads / p.kv_heads;
  const int SL = p.split_len;
  float *qr = smem;                  // [G][D]
  float *sc = qr + G * D;            // [G][SL]
  float *ck = sc + G * SL;           // [256]
  float *cv = ck + kMaxLevels;       // [256]
  float *red = cv + kMaxLevels;      // [4]

  const int split = blockIdx.x;
  const long bk = blockIdx.y;
  const int b = static_cast<int>(bk / p.kv_heads), kv = static_cast<int>(bk % p.kv_heads);
  const int t0 = split * SL;
  const int t1 = min(p.length, t0 + SL);
  const int n = max(0, t1 - t0);
  const long hq0 = static_cast<long>(b) * p.q_heads + static_cast<long>(kv) * G;

  for (int i = threadIdx.x; i < kMaxLevels; i += kBlock) {
    ck[i] = p.k_cent[i];
    cv[i] = p.v_cent[i];
  }
  const bool k_packed = p.k.mode == TQ_SIDE_PACKED;
  for (int i = threadIdx.x; i < G * D; i += kBlock) {
    const float x = h2f(p.q[hq0 * D + i]);
    qr[i] = k_packed ? x * sign_of(p.sign, i % D) : x;
  }
  __syncthreads();
  if (k_packed) {
    for (int s = 1; s < D; s <<= 1) {
      for (int i = threadIdx.x; i < G * D / 2; i += kBlock) {
        const int h = i / (D / 2), r = i % (D / 2);
        const int j = (r / s) * 2 * s + (r % s);
        const float a = qr[h * D + j], c = qr[h * D + j + s];
        qr[h * D + j] = a + c;
        qr[h * D + j + s] = a - c;
      }
      __syncthreads();
    }
  }
  // score(i) = n_i <H s q / sqrt(D), c> / sqrt(D), here in base-2 units.
  const float qscale = k_packed ? kLog2e / static_cast<float>(D) : kLog2e / sqrtf(static_cast<float>(D));
  for (int i = threadIdx.x; i < G * D; i += kBlock) qr[i] *= qscale;
  __syncthreads();

  for (int i = threadIdx.x; i < n * G; i += kBlock) {
    const int tok = i / G, h = i % G;
    const int t = t0 + tok;
    float acc = 0.0f;
    if (k_packed) {
      const uint32_t *row = p.k.codes + cache_row(p.pg, bk, t, p.capacity) * p.k.words;
      for (int j = 0; j < D; ++j) acc += qr[h * D + j] * ck[extract_code(row, p.k.bits, j)];
      acc *= p.k.norms[cache_row(p.pg, bk, t, p.capacity)];
    } else if (p.k.mode == TQ_SIDE_INT8) {
      // INT8 rows: q . code times the row's scale (original domain)
      const uint32_t *row = p.k.codes + cache_row(p.pg, bk, t, p.capacity) * p.k.words;
      for (int j = 0; j < D; ++j) acc += qr[h * D + j] * int8_at(row[j >> 2], j);
      acc *= p.k.norms[cache_row(p.pg, bk, t, p.capacity)];
    } else {
      const uint16_t *row = p.k.fp16 + cache_row(p.pg, bk, t, p.capacity) * D;
      for (int j = 0; j < D; ++j) acc += qr[h * D + j] * h2f(row[j]);
    }
    sc[h * SL + tok] = acc;
    if (p.scores) p.scores[(hq0 + h) * p.length + t] = acc * kLn2;
  }
  __syncthreads();

  const DecodeWorkspace lay = decode_workspace_layout(p.batch, p.q_heads, p.n_splits, D);
  float *ml = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + lay.ml_off);
  for (int h = 0; h < G; ++h) {
    float m = -INFINITY;
    for (int tok = threadIdx.x; tok < n; tok += kBlock) m = fmaxf(m, sc[h * SL + tok]);
    m = block_reduce(m, red, true);
    float l = 0.0f;
    for (int tok = threadIdx.x; tok < n; tok += kBlock) {
      const float e = (n > 0) ? exp2f(sc[h * SL + tok] - m) : 0.0f;
      sc[h * SL + tok] = e;
      l += e;
    }
    l = block_reduce(l, red, false);
    if (threadIdx.x == 0) {
      ml[((hq0 + h) * p.n_splits + split) * 2 + 0] = m;
      ml[((hq0 + h) * p.n_splits + split) * 2 + 1] = l;
    }
  }
  __syncthreads();

  float *orot = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + lay.orot_off);
  float *ohot = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + lay.ohot_off);
  for (int o = threadIdx.x; o < G * D; o += kBlock) {
    const int h = o / D, j = o % D;
    float rot = 0.0f, plain = 0.0f;
    for (int tok = 0; tok < n; ++tok) {
      const int t = t0 + tok;
      const float w = sc[h * SL + tok];
      // sparse-V: weight relative to the split's maximum below the threshold
      if (p.sparse_lg != -INFINITY && !(log2f(w) >= p.sparse_lg)) continue;
      const uint16_t *vrow = v_plain_row(p, bk, t);
      if (vrow) {
        plain += w * h2f(vrow[j]);
      } else if (p.v.mode == TQ_SIDE_INT8) {
        const uint32_t *row = p.v.codes + cache_row(p.pg, bk, t, p.capacity) * p.v.words;
        plain += w * p.v.norms[cache_row(p.pg, bk, t, p.capacity)] * int8_at(row[j >> 2], j);
      } else {
        const uint32_t *row = p.v.codes + cache_row(p.pg, bk, t, p.capacity) * p.v.words;
        rot += w * p.v.norms[cache_row(p.pg, bk, t, p.capacity)] * cv[extract_code(row, p.v.bits, j)];
      }
    }
    const long u = (hq0 + h) * p.n_splits + split;
    orot[u * D + j] = rot;
    ohot[u * D + j] = plain;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const DecodeParams p) {
  __shared__ float buf[D];
  const long bh = blockIdx.x;
  const int j = threadIdx.x;
  const DecodeWorkspace lay = decode_workspace_layout(p.batch, p.q_heads, p.n_splits, D);
  const float *ml = reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.ws) + lay.ml_off);
  const float *orot = reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.ws) + lay.orot_off);
  const float *ohot = reinterpret_cast<const float *>(reinterpret_cast<const char *>(p.ws) + lay.ohot_off);
  float M = -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, ml[(bh * p.n_splits + s) * 2]);
  float L = 0.0f, rot = 0.0f, plain = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < p.n_splits; ++s) {
      const long u = bh * p.n_splits + s;
      const float w = exp2f(ml[u * 2] - M);
      L += w * ml[u * 2 + 1];
      rot += w * orot[u * D + j];
      plain += w * ohot[u * D + j];
    }
  }
  buf[j] = rot;
  __syncthreads();
  for (int s = 1; s < D; s <<= 1) {
    float a = 0.0f, c = 0.0f;
    const bool low = (j & s) == 0;
    if (low) {
      a = buf[j];
      c = buf[j + s];
    }
    __syncthreads();
    if (low) {
      buf[j] = a + c;
      buf[j + s] = a - c;
    }
    __syncthreads();
  }
  const float o = buf[j] * sign_of(p.sign, j) / sqrtf(static_cast<float>(D));
  p.out[bh * D + j] = (L > 0.0f) ? (o + plain) / L : 0.0f;
}

template <int D>
hipError_t launch_d(const DecodeParams &p, hipStream_t stream) {
  const int G = p.q_heads / p.kv_heads;
  const size_t smem = sizeof(float) * (static_cast<size_t>(G) * D + static_cast<size_t>(G) * p.split_len +
                                       2 * kMaxLevels + 4);
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3(p.n_splits, p.batch * p.kv_heads), dim3(kBlock), smem,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(p.batch * p.q_heads), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_ref(const DecodeParams &p, hipStream_t stream) {
  switch (p.head_dim) {
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 256: return launch_d<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
