// Split-context decode attention from the packed cache on the matrix cores
// ("TurboQuant KV Cache Quantization in MLX-VLM", "How TurboQuant KV Cache
// Quantization Works": scores straight from the compressed representation;
// FAQ on dequantization: one stored rotation plus codebooks; mlxcel
// "TurboQuant KV cache", "Available modes": fp16 K with TurboQuant V and the
// delegated hot/cold V split).
//
// head_dim 128, 4-bit V codes, K packed (3 or 4 bits) or fp16, up to 16
// query heads per KV head.  Block = 4 waves; grid = (B * Hkv units) x splits.
// Each wave walks its share of the split in chunks of 32 positions:
//
//   score   v_mfma_f32_16x16x32_f16 with M = 16 positions, N = 16 (the G
//           query heads, rest padding), K = 32 coordinates.  A holds the
//           centroids of the position's codes, decoded two codes at a time
//           from pair tables in LDS (32 replicas of every 32-bit entry, one
//           per bank, so any index pattern reads without bank conflicts); B
//           holds R q, rotated once per block with 1/sqrt(d) and log2(e)
//           folded in.  Times the position's norm this is the base-2 logit.
//   softmax online per query head; the accumulators are only rescaled when
//           the running maximum grows by more than 2^8.
//   value   the same MFMA with M = 16 coordinates, N = 16 heads, K = 32
//           positions.  Each lane loads one code word of 8 positions and
//           transposes the 8 x 8 nibbles in registers, so it then holds one
//           coordinate of 8 positions; B holds p_i n_i (scaled by a power of
//           two so fp16 cannot overflow).  The sum stays in the rotated
//           domain; the fp16 hot window of a delegated V is a split of its
//           own that sums in the original domain.
//   precision  fp16 operands carry 11 bits, and the output of a diffuse
//           softmax is much smaller than the rows it averages, so plain fp16
//           leaves output errors near 1e-3.  Each fp16 operand that is not
//           exact is therefore a hi + lo pair (lo = the fp16 rounding of the
//           remainder): the score takes A_hi B_hi + A_lo B_hi + A_hi B_lo,
//           the value sum takes A_hi (P_hi + P_lo); fp16 K rows are exact.
//
// The 4 waves merge in LDS and write one partial (max, sum, accumulator) per
// query head with L2-coherent stores; the last block of a unit to arrive
// (atomic counter) merges the splits with L2-coherent loads, applies the
// inverse rotation diag(s) H / sqrt(d) once per head, adds the hot part and
// divides by the sum.
#include <math.h>

#include <algorithm>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;
constexpr int kRep = 32;          // pair-table replicas, one per LDS bank
constexpr int kMaxSplits = 256;   // splits per unit the merge can stage
constexpr float kRescale = 8.0f;  // lazy rescaling threshold (log2 units)

// Static LDS layout (32-bit words) per K width.
//   KB = 3: K hi [64 x 32] | K lo [64 x 32] | V hi [256 x 32] | codebooks | work
//   KB = 4: K/V hi [256 x 32] (one codebook) | K lo [256 x 16] | ... (the lo
//           reads then see 2-way bank conflicts; the table would not fit
//           otherwise)
//   KB = 0: V hi [256 x 32] | ...
template <int KB>
struct Lay {
  static constexpr int klo_rep = KB == 4 ? 16 : kRep;
  static constexpr int khi = 0;
  static constexpr int klo = KB == 3 ? 64 * kRep : (KB == 4 ? 256 * kRep : 0);
  static constexpr int vhi = KB == 3 ? 2 * 64 * kRep : 0;
  static constexpr int end_tables = KB == 3 ? 2 * 64 * kRep + 256 * kRep
                                            : (KB == 4 ? 256 * kRep + 256 * 16 : 256 * kRep);
  static constexpr int cent = end_tables;
  static constexpr int work = cent + 2 * kMaxLevels;
};

__device__ __forceinline__ float4_t mma(const half8_t a, const half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  return static_cast<uint32_t>(f2h(lo)) | (static_cast<uint32_t>(f2h(hi)) << 16);
}

// hi and lo halves of a float pair: hi = fp16(x), lo = fp16(x - hi).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  const float h0 = h2f(f2h(x0)), h1 = h2f(f2h(x1));
  hi = pack_half2(h0, h1);
  lo = pack_half2(x0 - h0, x1 - h1);
}

struct Frag {
  half8_t hi, lo;
};

__device__ __forceinline__ uint32_t ld(const uint32_t *lds, int word) { return lds[word]; }

// Decode the 32 coordinates [32 g, 32 g + 32) of one position into four K
// fragments (octet c -> fragment c) from the pair tables.
template <int KB>
__device__ __forceinline__ void decode_k(const uint32_t (&w)[4], const uint32_t *lds, int rep_hi,
                                         int rep_lo, Frag (&a)[4]) {
  using L = Lay<KB>;
  uint32_t idx[16];
  if (KB == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int k = 0; k < 4; ++k) idx[4 * c + k] = (w[c] >> (8 * k)) & 0xffu;
    }
  } else {
    // 96 bits = 16 six-bit pairs; pairs 5 and 10 straddle a word boundary.
#pragma unroll
    for (int k = 0; k < 5; ++k) idx[k] = (w[0] >> (6 * k)) & 63u;
    idx[5] = ((w[0] >> 30) | (w[1] << 2)) & 63u;
#pragma unroll
    for (int k = 6; k < 10; ++k) idx[k] = (w[1] >> (6 * k - 32)) & 63u;
    idx[10] = ((w[1] >> 28) | (w[2] << 4)) & 63u;
#pragma unroll
    for (int k = 11; k < 16; ++k) idx[k] = (w[2] >> (6 * k - 64)) & 63u;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = static_cast<int>(idx[4 * c + k]);
      h[k] = ld(lds, L::khi + e * kRep + rep_hi);
      l[k] = ld(lds, L::klo + e * L::klo_rep + rep_lo);
    }
    a[c].hi = as_half8(h[0], h[1], h[2], h[3]);
    a[c].lo = as_half8(l[0], l[1], l[2], l[3]);
  }
}

// 8 x 8 nibble transpose: x[s] holds codes 8w .. 8w+7 of position s; after
// it, x[p] holds coordinate 8w + p of positions 0 .. 7 (nibble s).
__device__ __forceinline__ void transpose8(uint32_t (&x)[8]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t a = x[s], b = x[s + 4];
    x[s] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    x[s + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s = (q & 1) + 4 * (q >> 1);
    const uint32_t a = x[s], b = x[s + 2];
    x[s] = __builtin_amdgcn_perm(b, a, 0x06020400u);
    x[s + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
  }
#pragma unroll
  for (int s = 0; s < 8; s += 2) {
    const uint32_t a = x[s], b = x[s + 1];
    x[s] = (a & 0x0f0f0f0fu) | ((b << 4) & 0xf0f0f0f0u);
    x[s + 1] = ((a >> 4) & 0x0f0f0f0fu) | (b & 0xf0f0f0f0u);
  }
}

__device__ __forceinline__ float max16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float sum16_32(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

__device__ __forceinline__ float block_max(float x, float *red) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float x, float *red) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Smallest power of two >= x (x > 0), as a float; 1 for x <= 0.
__device__ __forceinline__ float pow2_ceil(float x) {
  if (!(x > 0.0f)) return 1.0f;
  int e;
  const float m = frexpf(x, &e);  // x = m 2^e, m in [0.5, 1)
  return ldexpf(1.0f, m == 0.5f ? e - 1 : e);
}

__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KB>
struct Wave {
  // per-lane constants
  int col, grp, rep, rep_lo;
  const uint32_t *lds;
  Frag bq[4];
  // per-unit bases
  const uint32_t *kcodes;
  const uint16_t *k16;
  const float *knorm;
  const uint32_t *vcodes;
  const float *vnorm;
  const uint16_t *ring;
  int hot_len, G;
  float vscale;
  // running state
  float m_run, l_run;
  float4_t accv[8];

  // One chunk of 32 positions starting at t0; positions >= we are masked
  // (only in the tail chunk).
  template <bool TAIL, bool HOT>
  __device__ __forceinline__ void chunk(int t0, int we, float *scores, long score_row, int length) {
    // ---- scores: A rows are positions t0 + 16 m + col
    float4_t acc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int tr = TAIL ? min(t0 + 16 * m + col, we - 1) : t0 + 16 * m + col;
      acc[m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (KB) {
        uint32_t w[4];
        if (KB == 4) {
          const uint4 w4 = *reinterpret_cast<const uint4 *>(kcodes + tr * 16 + 4 * grp);
          w[0] = w4.x; w[1] = w4.y; w[2] = w4.z; w[3] = w4.w;
        } else {
          const uint32_t *src = kcodes + tr * 12 + 3 * grp;
          w[0] = src[0]; w[1] = src[1]; w[2] = src[2]; w[3] = 0u;
        }
        Frag a[4];
        decode_k<KB>(w, lds, rep, rep_lo, a);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[m] = mma(a[c].hi, bq[c].hi, acc[m]);
          acc[m] = mma(a[c].lo, bq[c].hi, acc[m]);
          acc[m] = mma(a[c].hi, bq[c].lo, acc[m]);
        }
      } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(k16 + tr * D + 32 * grp);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 v = src[c];
          const half8_t a = as_half8(v.x, v.y, v.z, v.w);
          acc[m] = mma(a, bq[c].hi, acc[m]);
          acc[m] = mma(a, bq[c].lo, acc[m]);
        }
      }
    }
    // ---- lane holds positions t0 + 16 m + 4 grp + r for head col
    float s[8], vn[8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int base = t0 + 16 * m + 4 * grp;
      float4 nk = make_float4(1.0f, 1.0f, 1.0f, 1.0f), nv = nk;
      if (TAIL) {
        float kk[4], vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tc = min(base + r, we - 1);
          kk[r] = KB ? knorm[tc] : 1.0f;
          vv[r] = HOT ? 1.0f : vnorm[tc];
        }
        nk = make_float4(kk[0], kk[1], kk[2], kk[3]);
        nv = make_float4(vv[0], vv[1], vv[2], vv[3]);
      } else {
        if (KB) nk = *reinterpret_cast<const float4 *>(knorm + base);
        if (!HOT) nv = *reinterpret_cast<const float4 *>(vnorm + base);
      }
      const float nks[4] = {nk.x, nk.y, nk.z, nk.w};
      const float nvs[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = acc[m][r] * nks[r];
        s[4 * m + r] = (TAIL && base + r >= we) ? -INFINITY : x;
        vn[4 * m + r] = HOT ? 1.0f : nvs[r] * vscale;
      }
    }
    if (scores && col < G) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = t0 + 16 * (i >> 2) + 4 * grp + (i & 3);
        if (!TAIL || t < we) scores[score_row * length + t] = s[i] * kLn2;
      }
    }
    // ---- online softmax with lazy rescaling
    float cmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, s[i]);
    cmax = max16_32(cmax);
    const bool grow = cmax > m_run + kRescale;
    if (__ballot(grow)) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) accv[i] *= alpha;
    }
    uint32_t bh[4], bl[4];
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float p0 = __builtin_amdgcn_exp2f(s[i] - m_run);
      float p1 = __builtin_amdgcn_exp2f(s[i + 1] - m_run);
      if (TAIL) {
        p0 = (s[i] == -INFINITY) ? 0.0f : p0;
        p1 = (s[i + 1] == -INFINITY) ? 0.0f : p1;
      }
      lsum += p0 + p1;
      split_pair(p0 * vn[i], p1 * vn[i + 1], bh[i / 2], bl[i / 2]);
    }
    l_run += lsum;
    const half8_t bvh = as_half8(bh[0], bh[1], bh[2], bh[3]);
    const half8_t bvl = as_half8(bl[0], bl[1], bl[2], bl[3]);

    // ---- values
    if (!HOT) {
      // code word `col` of positions t0 + 4 grp + r and t0 + 16 + 4 grp + r
      uint32_t x[8];
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        int t = t0 + 16 * (s8 >> 2) + 4 * grp + (s8 & 3);
        if (TAIL) t = min(t, we - 1);
        x[s8] = vcodes[t * 16 + col];
      }
      transpose8(x);
      using L = Lay<KB>;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t y = x[q];
        const half8_t a = as_half8(ld(lds, L::vhi + static_cast<int>(y & 0xffu) * kRep + rep),
                                   ld(lds, L::vhi + static_cast<int>((y >> 8) & 0xffu) * kRep + rep),
                                   ld(lds, L::vhi + static_cast<int>((y >> 16) & 0xffu) * kRep + rep),
                                   ld(lds, L::vhi + static_cast<int>(y >> 24) * kRep + rep));
        accv[q] = mma(a, bvh, accv[q]);
        accv[q] = mma(a, bvl, accv[q]);
      }
    } else {
      // fp16 ring rows: tile q covers coordinates 16 q + col
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t u[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          uint32_t h2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int s8 = 2 * s2 + e;
            const int t = min(t0 + 16 * (s8 >> 2) + 4 * grp + (s8 & 3), we - 1);
            h2[e] = ring[(t % hot_len) * D + 16 * q + col];
          }
          u[s2] = h2[0] | (h2[1] << 16);
        }
        const half8_t a = as_half8(u[0], u[1], u[2], u[3]);
        accv[q] = mma(a, bvh, accv[q]);
        accv[q] = mma(a, bvl, accv[q]);
      }
    }
  }
};

template <int KB>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(const DecodeParams p) {
  using L = Lay<KB>;
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = p.q_heads / p.kv_heads;
  float *cent = reinterpret_cast<float *>(lds + L::cent);
  float *work = reinterpret_cast<float *>(lds + L::work);  // rotation; merge scratch
  const int wmax = max(kWaves * G * (D + 2), G * kMaxSplits + 2 * G * D + G);
  float *red = work + wmax;                                   // [4] block reductions
  int *flag = reinterpret_cast<int *>(red + 4);

  const int nsplit = p.n_cold_splits + p.n_hot_splits;
  const int unit = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  const int b = unit / p.kv_heads;
  const int kv = unit % p.kv_heads;
  const long hq0 = static_cast<long>(b) * p.q_heads + static_cast<long>(kv) * G;
  const bool hot = split >= p.n_cold_splits;
  int s0, s1;
  if (!hot) {
    s0 = split * p.cold_split_len;
    s1 = min(p.cold_len, s0 + p.cold_split_len);
  } else {
    s0 = p.cold_len + (split - p.n_cold_splits) * p.hot_split_len;
    s1 = min(p.length, s0 + p.hot_split_len);
  }
  const int span = max(0, s1 - s0);
  const int per = ((span + kWaves - 1) / kWaves + kChunk - 1) / kChunk * kChunk;
  const int ws = s0 + wave * per;
  const int we = min(s1, ws + per);

  // ---- prologue: codebooks, pair tables, rotated query ------------------
  for (int i = threadIdx.x; i < kMaxLevels; i += kThreads) {
    cent[i] = p.k_cent[i];
    cent[kMaxLevels + i] = p.v_cent[i];
  }
  constexpr bool k_packed = KB != 0;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const float x = h2f(p.q[hq0 * D + i]);
    work[i] = k_packed ? x * sign_of(p.sign, i % D) : x;
  }
  __syncthreads();
  // value table (for KB = 4 also the K hi table: one codebook)
  for (int i = threadIdx.x; i < 256 * kRep; i += kThreads) {
    const int e = i / kRep;
    lds[L::vhi + i] = pack_half2(cent[kMaxLevels + (e & 15)], cent[kMaxLevels + (e >> 4)]);
  }
  if (KB == 3) {
    for (int i = threadIdx.x; i < 64 * kRep; i += kThreads) {
      const int e = i / kRep;
      uint32_t h, l;
      split_pair(cent[e & 7], cent[e >> 3], h, l);
      lds[L::khi + i] = h;
      lds[L::klo + i] = l;
    }
  } else if (KB == 4) {
    for (int i = threadIdx.x; i < 256 * L::klo_rep; i += kThreads) {
      const int e = i / L::klo_rep;
      uint32_t h, l;
      split_pair(cent[e & 15], cent[e >> 4], h, l);
      lds[L::klo + i] = l;
    }
  }
  if (k_packed) {
    for (int s = 1; s < D; s <<= 1) {
      for (int i = threadIdx.x; i < G * D / 2; i += kThreads) {
        const int h = i / (D / 2), r = i % (D / 2);
        const int j = (r / s) * 2 * s + (r % s);
        const float a = work[h * D + j], c = work[h * D + j + s];
        work[h * D + j] = a + c;
        work[h * D + j + s] = a - c;
      }
      __syncthreads();
    }
  }
  __syncthreads();

  Wave<KB> W;
  W.col = lane & 15;
  W.grp = lane >> 4;
  W.rep = lane & (kRep - 1);
  W.rep_lo = lane & (L::klo_rep - 1);
  W.lds = lds;
  W.G = G;
  {
    const float qscale = k_packed ? kLog2e / static_cast<float>(D) : kLog2e / sqrtf(static_cast<float>(D));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = 32 * W.grp + 8 * c + 2 * s;
        h[s] = l[s] = 0u;
        if (W.col < G) split_pair(work[W.col * D + j] * qscale, work[W.col * D + j + 1] * qscale, h[s], l[s]);
      }
      W.bq[c].hi = as_half8(h[0], h[1], h[2], h[3]);
      W.bq[c].lo = as_half8(l[0], l[1], l[2], l[3]);
    }
  }
  const long rowbase = static_cast<long>(unit) * p.capacity;
  W.kcodes = KB ? p.k.codes + rowbase * (KB == 4 ? 16 : 12) : nullptr;
  W.k16 = KB ? nullptr : p.k.fp16 + rowbase * D;
  W.knorm = KB ? p.k.norms + rowbase : nullptr;
  W.vcodes = p.v.codes + rowbase * 16;
  W.vnorm = p.v.norms + rowbase;
  W.hot_len = p.v.hot > 0 ? p.v.hot : 1;
  W.ring = (p.v.mode == TQ_SIDE_DELEGATED) ? p.v.fp16 + static_cast<long>(unit) * p.v.hot * D : nullptr;
  W.m_run = -INFINITY;
  W.l_run = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) W.accv[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // V norm scale of this wave: a power of two that keeps p n below 2^9.
  W.vscale = 1.0f;
  if (!hot) {
    float nmax = 0.0f;
    for (int t = ws + lane; t < we; t += 64) nmax = fmaxf(nmax, W.vnorm[t]);
    for (int m = 32; m >= 1; m >>= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, m));
    W.vscale = 1.0f / pow2_ceil(nmax);
  }

  // ---- main loop ------------------------------------------------------
  const long score_row = hq0 + W.col;
  const int full_end = ws + (max(0, we - ws) / kChunk) * kChunk;
  if (!hot) {
    for (int t0 = ws; t0 < full_end; t0 += kChunk) W.template chunk<false, false>(t0, we, p.scores, score_row, p.length);
    if (full_end < we) W.template chunk<true, false>(full_end, we, p.scores, score_row, p.length);
  } else {
    for (int t0 = ws; t0 < we; t0 += kChunk) W.template chunk<true, true>(t0, we, p.scores, score_row, p.length);
  }

  // ---- merge the waves of this block ------------------------------------
  const float l_wave = sum16_32(W.l_run);
  __syncthreads();  // rotation buffer no longer needed
  float *mw = work + wave * G * (D + 2);
  if (W.col < G) {
    float *slot = mw + W.col * (D + 2);
    if (W.grp == 0) {
      slot[0] = W.m_run;
      slot[1] = l_wave;
    }
    const float inv = 1.0f / W.vscale;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int coord = hot ? 16 * q + 4 * W.grp + r : 8 * (4 * W.grp + r) + q;
        slot[2 + coord] = W.accv[q][r] * inv;
      }
    }
  }
  __syncthreads();
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + p.ws_part_off);
  float *mypart = part + (static_cast<long>(unit) * nsplit + split) * G * (D + 2);
  for (int i = threadIdx.x; i < G * (D + 2); i += kThreads) {
    const int h = i / (D + 2), j = i % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, work[(w * G + h) * (D + 2)]);
    float v;
    if (M == -INFINITY) {
      v = (j == 0) ? -INFINITY : 0.0f;
    } else if (j == 0) {
      v = M;
    } else {
      v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw_ = work[(w * G + h) * (D + 2)];
        const float sc = (mw_ == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw_ - M);
        v += sc * work[(w * G + h) * (D + 2) + j];
      }
    }
    store_coherent(mypart + i, v);
  }

  // ---- the last block of the unit merges the splits ----------------------
  // The partials above are L2-coherent stores; once they have completed
  // (s_waitcnt), the arrival counter is bumped.  The last arrival reads all
  // partials with L2-coherent loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(p.counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == static_cast<unsigned>(nsplit - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;

  const float *up = part + static_cast<long>(unit) * nsplit * G * (D + 2);
  float *wts = work;                   // [G][kMaxSplits] split weights 2^(m_s - M)
  float *rot = work + G * kMaxSplits;  // [G][D] rotated-domain sum
  float *pln = rot + G * D;            // [G][D] plain (hot) sum
  float *Ls = pln + G * D;             // [G] total sums
  for (int h = 0; h < G; ++h) {
    float m = -INFINITY;
    for (int sp = threadIdx.x; sp < nsplit; sp += kThreads) m = fmaxf(m, load_coherent(up + (sp * G + h) * (D + 2)));
    const float M = block_max(m, red);
    float l = 0.0f;
    for (int sp = threadIdx.x; sp < nsplit; sp += kThreads) {
      const float ms = load_coherent(up + (sp * G + h) * (D + 2));
      const float w = (ms == -INFINITY || M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
      wts[h * kMaxSplits + sp] = w;
      l += w * load_coherent(up + (sp * G + h) * (D + 2) + 1);
    }
    const float Lh = block_sum(l, red);
    if (threadIdx.x == 0) Ls[h] = Lh;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, j = i % D;
    float r = 0.0f, q = 0.0f;
    for (int sp = 0; sp < p.n_cold_splits; ++sp)
      r += wts[h * kMaxSplits + sp] * load_coherent(up + (sp * G + h) * (D + 2) + 2 + j);
    for (int sp = p.n_cold_splits; sp < nsplit; ++sp)
      q += wts[h * kMaxSplits + sp] * load_coherent(up + (sp * G + h) * (D + 2) + 2 + j);
    rot[i] = r;
    pln[i] = q;
  }
  __syncthreads();
  for (int s = 1; s < D; s <<= 1) {
    for (int i = threadIdx.x; i < G * D / 2; i += kThreads) {
      const int h = i / (D / 2), r = i % (D / 2);
      const int j = (r / s) * 2 * s + (r % s);
      const float a = rot[h * D + j], c = rot[h * D + j + s];
      rot[h * D + j] = a + c;
      rot[h * D + j + s] = a - c;
    }
    __syncthreads();
  }
  const float rs = 1.0f / sqrtf(static_cast<float>(D));
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, j = i % D;
    const float Lh = Ls[h];
    const float o = rot[i] * sign_of(p.sign, j) * rs + pln[i];
    p.out[(hq0 + h) * D + j] = (Lh > 0.0f) ? o / Lh : 0.0f;
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KB>
size_t lds_bytes(int G) {
  using L = Lay<KB>;
  const size_t merge = size_t(kWaves) * G * (D + 2);
  const size_t combine = size_t(G) * kMaxSplits + 2 * size_t(G) * D + G;
  return 4 * (L::work + std::max(merge, combine) + 4 + 1);
}

}  // namespace

size_t decode_mfma_lds_bytes(int k_bits, bool share_lut, int G) {
  (void)share_lut;
  switch (k_bits) {
    case 0: return lds_bytes<0>(G);
    case 3: return lds_bytes<3>(G);
    case 4: return lds_bytes<4>(G);
    default: return ~size_t(0);
  }
}

bool decode_mfma_supported(const DecodeParams &p) {
  const int G = p.q_heads / p.kv_heads;
  if (p.head_dim != D || G > 16) return false;
  if (!(p.v.mode == TQ_SIDE_PACKED || p.v.mode == TQ_SIDE_DELEGATED) || p.v.bits != 4) return false;
  int kb;
  if (p.k.mode == TQ_SIDE_FP16) {
    kb = 0;
  } else if (p.k.mode == TQ_SIDE_PACKED && p.k.bits == 3) {
    kb = 3;
  } else if (p.k.mode == TQ_SIDE_PACKED && p.k.bits == 4 && p.share_lut) {
    kb = 4;  // K and V share one 4-bit codebook table
  } else {
    return false;
  }
  return decode_mfma_lds_bytes(kb, p.share_lut != 0, G) <= 65536;
}

int decode_mfma_max_splits() { return kMaxSplits; }

hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t stream) {
  const int G = p.q_heads / p.kv_heads;
  const int kb = p.k.mode == TQ_SIDE_PACKED ? p.k.bits : 0;
  const size_t lds = decode_mfma_lds_bytes(kb, p.share_lut != 0, G);
  const int nsplit = p.n_cold_splits + p.n_hot_splits;
  if (nsplit > kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.batch * p.kv_heads * nsplit));
  switch (kb) {
    case 0: hipLaunchKernelGGL(decode_mfma_kernel<0>, grid, dim3(kThreads), lds, stream, p); break;
    case 3: hipLaunchKernelGGL(decode_mfma_kernel<3>, grid, dim3(kThreads), lds, stream, p); break;
    case 4: hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(kThreads), lds, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
