// Split-context decode attention from the packed cache on the matrix cores
// ("TurboQuant KV Cache Quantization in MLX-VLM", "How TurboQuant KV Cache
// Quantization Works": scores straight from the compressed representation;
// FAQ on dequantization: one stored rotation plus codebooks; mlxcel
// "TurboQuant KV cache", "Available modes": fp16 K with TurboQuant V and the
// delegated hot/cold V split).
//
// head_dim 128, 4-bit V codes, K packed (3 or 4 bits) or fp16, up to 8 (fp16
// K) or 4 (packed K) query heads per KV head.  Grid = (B * Hkv units) x
// splits, about one 8-wave block per compute unit.  A block issues its first
// loads, builds its lookup tables and rotated query while they are in
// flight, then each wave walks its share of the split in chunks of 32
// positions, loading chunk i + 1 while it computes chunk i:
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
//           coordinate of 8 positions; B holds p_i n_i times a power of two
//           that keeps fp16 in range (lowered lazily when a larger norm
//           arrives).  The sum stays in the rotated domain.
//   precision  fp16 operands carry 11 bits, and the output of a diffuse
//           softmax is much smaller than the rows it averages, so plain fp16
//           leaves output errors near 1e-3.  Each fp16 operand that is not
//           exact is therefore a hi + lo pair (lo = the fp16 rounding of the
//           remainder): the score takes A_hi B_hi + A_lo B_hi + A_hi B_lo,
//           the value sum takes A_hi (P_hi + P_lo); fp16 K rows are exact.
//
// The 8 waves merge in LDS (over the dead tables) and write one partial
// (max, sum, accumulator) per query head with L2-coherent stores; the last
// block of a unit to arrive (atomic counter) attends over the fp16 hot window
// of a delegated V (original domain), merges the splits with L2-coherent
// loads, applies the inverse rotation diag(s) H / sqrt(d) once per head, adds
// the hot part and divides by the sum.
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
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;
constexpr int kRep = 32;          // pair-table replicas, one per LDS bank
constexpr int kMaxSplits = 256;   // splits per unit (bounded by the host)
constexpr float kRescale = 8.0f;  // lazy rescaling threshold (log2 units)
constexpr float kVscaleMax = 1099511627776.0f;  // 2^40: start and ceiling of the V scale

// Static LDS layout (32-bit words) per K width.  Tables hold fp16 pairs for
// a code pair index e (first code in the low bits); replica r of entry e sits
// at word e * reps + r, so lane r of each 32-lane half reads its own bank.
// The lo tables start one word past a 64-word boundary so the compiler cannot
// fuse a hi and a lo read into one two-address instruction (which would land
// hi and lo in adjacent registers and cost register copies).
//   KB = 3: K hi [64 x 32] | K lo [64 x 32] | V hi [256 x 32] | codebooks | q
//   KB = 4: K/V hi [256 x 32] (one codebook) | K lo [256 x 16] | ... (2-way
//           bank conflicts on the lo reads; a 32-replica lo table would not
//           fit in 64 KB)
//   KB = 0: V hi [256 x 32] | codebooks | q
// After the main loop the whole area is reused for the merges.
template <int KB>
struct Lay {
  static constexpr int max_g = KB == 0 ? 8 : 4;  // query heads per KV head supported
  static constexpr int klo_rep = KB == 4 ? 16 : kRep;
  static constexpr int khi = 0;
  static constexpr int klo = KB == 3 ? 64 * kRep + 1 : (KB == 4 ? 256 * kRep + 1 : 0);
  static constexpr int vhi = KB == 3 ? 2 * 64 * kRep + 2 : 0;
  static constexpr int end_tables = KB == 3 ? vhi + 256 * kRep
                                            : (KB == 4 ? klo + 256 * 16 : 256 * kRep);
  static constexpr int cent = (end_tables + 3) & ~3;
  static constexpr int qwork = cent + 2 * kMaxLevels;           // [G][D] rotated query
  static constexpr int red = qwork + max_g * D;                  // [16] reductions, flag
  static constexpr int total = red + 16;
  static constexpr int merge_words = kWaves * max_g * (D + 2);  // reuses [0, red)
  static_assert(merge_words + max_g * (D + 2) <= red, "wave slots + hot partial must fit in the tables");
  static_assert(4 * total <= 65536, "LDS budget");
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

// LDS word at byte address `addr` plus a compile-time byte offset.
template <int OFF>
__device__ __forceinline__ uint32_t lds_at(const uint32_t *lds, uint32_t addr) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lds) + addr + OFF);
}

// Byte address of table entry (v >> sh) & mask for a table with 32
// replicas: ((v >> sh) & mask) * 128 + rep * 4, i.e. shift so the index
// lands at bit 7, mask, and OR the lane's replica offset.
template <int SH, uint32_t MASK>
__device__ __forceinline__ uint32_t taddr(uint32_t v, uint32_t rep4) {
  const uint32_t x = (SH >= 7) ? (v >> (SH - 7)) : (v << (7 - SH));
  return (x & (MASK << 7)) | rep4;
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

// Buffer resource over [base, base + bytes): loads past the end read 0.
constexpr int kBufFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes > 0 ? bytes : 0, kBufFlags);
}

__device__ __forceinline__ float4 bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, int imm) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + imm, 0, 0);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// Global-memory data of one chunk of 32 positions for one lane.
template <int KB>
struct ChunkData {
  static constexpr int kw = KB == 0 ? 16 : (KB == 4 ? 4 : 3);  // K dwords per M-tile
  uint32_t k[2][kw];   // K words (packed) or fp16 row piece, M-tiles 0 and 1
  float4 kn[2];        // K norms of positions t0 + 16 m + 4 grp .. + 3
  uint32_t v[8];       // V code word `col` of the 8 positions of this K group
  float4 vn[2];        // V norms, same positions as kn
};

template <int KB>
struct Wave {
  // per-lane constants
  int col, grp;
  uint32_t rep4, rep4lo;
  uint32_t koff, knoff, voff;   // lane byte offsets inside a chunk
  const uint32_t *lds;
  Frag bq[4];
  // per-unit bases
  const char *kbase;   // K codes or fp16 rows of this unit
  const char *knbase;  // K norms
  const char *vbase;   // V codes
  const char *vnbase;  // V norms
  const uint16_t *ring;
  int capacity, hot_len, G;
  float vscale;        // power of two, n vscale <= 32 for every norm seen, so
                       // p n vscale < 2^13 fits fp16 (lowered as norms grow)
  // running state
  float m_run, l_run;
  float4_t accv[8];

  static constexpr int kRowBytes = KB == 0 ? 2 * D : (KB == 4 ? 64 : 48);

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) accv[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  __device__ __forceinline__ void load(int t0, ChunkData<KB> &c) const {
    // rows [t0, t0 + 32) at most; rows past the unit's capacity read 0
    const int rows = min(capacity - t0, kChunk);
    const auto rk = rsrc(kbase + static_cast<long>(t0) * kRowBytes, rows * kRowBytes);
    const auto rkn = rsrc(knbase + static_cast<long>(t0) * 4, rows * 4);
    const auto rv = rsrc(vbase + static_cast<long>(t0) * 64, rows * 64);
    const auto rvn = rsrc(vnbase + static_cast<long>(t0) * 4, rows * 4);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mo = m * 16 * kRowBytes;
      if (KB == 3) {
        typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
        const u32x3_t w = __builtin_amdgcn_raw_buffer_load_b96(rk, koff + mo, 0, 0);
        c.k[m][0] = w[0]; c.k[m][1] = w[1]; c.k[m][2] = w[2];
      } else {
#pragma unroll
        for (int i = 0; i < ChunkData<KB>::kw; i += 4) {
          const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + mo + 4 * i, 0, 0);
          c.k[m][i] = w[0]; c.k[m][i + 1] = w[1]; c.k[m][i + 2] = w[2]; c.k[m][i + 3] = w[3];
        }
      }
      if (KB) c.kn[m] = bload4f(rkn, knoff, 64 * m);
      c.vn[m] = bload4f(rvn, knoff, 64 * m);
    }
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      c.v[s8] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff + (16 * (s8 >> 2) + (s8 & 3)) * 64, 0, 0);
  }

  // Scores of the chunk (lane: positions t0 + 16 m + 4 grp + r, head col).
  __device__ __forceinline__ void score(const ChunkData<KB> &c, float (&s)[8]) const {
    using L = Lay<KB>;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (KB == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const half8_t a = as_half8(c.k[m][4 * q], c.k[m][4 * q + 1], c.k[m][4 * q + 2], c.k[m][4 * q + 3]);
          acc = mma(a, bq[q].hi, acc);
          acc = mma(a, bq[q].lo, acc);
        }
      } else {
        uint32_t ad[16];   // byte addresses of the 16 code pairs (32-replica tables)
        uint32_t adl[16];  // same in the lo table
        if (KB == 3) {
          const uint32_t w0 = c.k[m][0], w1 = c.k[m][1], w2 = c.k[m][2];
          ad[0] = taddr<0, 63>(w0, rep4);
          ad[1] = taddr<6, 63>(w0, rep4);
          ad[2] = taddr<12, 63>(w0, rep4);
          ad[3] = taddr<18, 63>(w0, rep4);
          ad[4] = taddr<24, 63>(w0, rep4);
          ad[5] = taddr<0, 63>(__builtin_amdgcn_alignbit(w1, w0, 30), rep4);
          ad[6] = taddr<4, 63>(w1, rep4);
          ad[7] = taddr<10, 63>(w1, rep4);
          ad[8] = taddr<16, 63>(w1, rep4);
          ad[9] = taddr<22, 63>(w1, rep4);
          ad[10] = taddr<0, 63>(__builtin_amdgcn_alignbit(w2, w1, 28), rep4);
          ad[11] = taddr<2, 63>(w2, rep4);
          ad[12] = taddr<8, 63>(w2, rep4);
          ad[13] = taddr<14, 63>(w2, rep4);
          ad[14] = taddr<20, 63>(w2, rep4);
          ad[15] = taddr<26, 63>(w2, rep4);
#pragma unroll
          for (int k = 0; k < 16; ++k) adl[k] = ad[k];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = c.k[m][q];
            ad[4 * q + 0] = taddr<0, 255>(w, rep4);
            ad[4 * q + 1] = taddr<8, 255>(w, rep4);
            ad[4 * q + 2] = taddr<16, 255>(w, rep4);
            ad[4 * q + 3] = taddr<24, 255>(w, rep4);
#pragma unroll
            for (int k = 0; k < 4; ++k) adl[4 * q + k] = ((ad[4 * q + k] >> 1) & 0x3fc0u) | rep4lo;
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const half8_t ah = as_half8(lds_at<4 * L::khi>(lds, ad[4 * q]), lds_at<4 * L::khi>(lds, ad[4 * q + 1]),
                                      lds_at<4 * L::khi>(lds, ad[4 * q + 2]), lds_at<4 * L::khi>(lds, ad[4 * q + 3]));
          const half8_t al = as_half8(lds_at<4 * L::klo>(lds, adl[4 * q]), lds_at<4 * L::klo>(lds, adl[4 * q + 1]),
                                      lds_at<4 * L::klo>(lds, adl[4 * q + 2]), lds_at<4 * L::klo>(lds, adl[4 * q + 3]));
          acc = mma(ah, bq[q].hi, acc);
          acc = mma(al, bq[q].hi, acc);
          acc = mma(ah, bq[q].lo, acc);
        }
      }
      const float nk[4] = {c.kn[m].x, c.kn[m].y, c.kn[m].z, c.kn[m].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * m + r] = KB ? acc[r] * nk[r] : acc[r];
    }
  }

  // Online softmax update (lazy: accumulators are rescaled only when the
  // running maximum grows by more than 2^8); returns the value-MFMA B
  // operands p n vscale as hi/lo fp16.
  template <bool TAIL>
  __device__ __forceinline__ void softmax(float (&s)[8], const float (&vn)[8], half8_t &bvh, half8_t &bvl) {
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
    bvh = as_half8(bh[0], bh[1], bh[2], bh[3]);
    bvl = as_half8(bl[0], bl[1], bl[2], bl[3]);
  }

  // Keep n vscale <= 32 for the norms of this chunk: if a larger norm shows
  // up, lower vscale (a power of two) and the accumulators with it.
  __device__ __forceinline__ void fit_vscale(const float (&v4)[8]) {
    float lm = v4[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) lm = fmaxf(lm, v4[i]);
    if (__ballot(lm * vscale > 32.0f)) {
      for (int m = 32; m >= 1; m >>= 1) lm = fmaxf(lm, __shfl_xor(lm, m));
      const float nv = fminf(32.0f / pow2_ceil(lm), kVscaleMax);
      const float f = nv / vscale;
      vscale = nv;
#pragma unroll
      for (int i = 0; i < 8; ++i) accv[i] *= f;
    }
  }

  // Packed values: transpose the 8 code words and accumulate 8 tiles.
  __device__ __forceinline__ void values(const ChunkData<KB> &c, const half8_t bvh, const half8_t bvl) {
    using L = Lay<KB>;
    uint32_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = c.v[i];
    transpose8(x);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t y = x[q];
      const half8_t a = as_half8(lds_at<4 * L::vhi>(lds, taddr<0, 255>(y, rep4)),
                                 lds_at<4 * L::vhi>(lds, taddr<8, 255>(y, rep4)),
                                 lds_at<4 * L::vhi>(lds, taddr<16, 255>(y, rep4)),
                                 lds_at<4 * L::vhi>(lds, taddr<24, 255>(y, rep4)));
      accv[q] = mma(a, bvh, accv[q]);
      accv[q] = mma(a, bvl, accv[q]);
    }
  }

  // One chunk of packed positions [t0, t0 + 32); positions >= we are masked.
  template <bool TAIL>
  __device__ __forceinline__ void cold_chunk(int t0, int we, const ChunkData<KB> &c, float *scores,
                                             long score_row, int length) {
    float s[8], vn[8];
    score(c, s);
    const float v4[8] = {c.vn[0].x, c.vn[0].y, c.vn[0].z, c.vn[0].w, c.vn[1].x, c.vn[1].y, c.vn[1].z, c.vn[1].w};
    fit_vscale(v4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vn[i] = v4[i] * vscale;
      if (TAIL && t0 + 16 * (i >> 2) + 4 * grp + (i & 3) >= we) s[i] = -INFINITY;
    }
    if (scores && col < G) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = t0 + 16 * (i >> 2) + 4 * grp + (i & 3);
        if (!TAIL || t < we) scores[score_row * length + t] = s[i] * kLn2;
      }
    }
    half8_t bvh, bvl;
    softmax<TAIL>(s, vn, bvh, bvl);
    values(c, bvh, bvl);
  }

  // One chunk of the fp16 hot window (delegated V), positions >= we masked.
  __device__ __forceinline__ void hot_chunk(int t0, int we, const ChunkData<KB> &c, float *scores,
                                            long score_row, int length) {
    float s[8];
    const float vn[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
    score(c, s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (t0 + 16 * (i >> 2) + 4 * grp + (i & 3) >= we) s[i] = -INFINITY;
    if (scores && col < G) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = t0 + 16 * (i >> 2) + 4 * grp + (i & 3);
        if (t < we) scores[score_row * length + t] = s[i] * kLn2;
      }
    }
    half8_t bvh, bvl;
    softmax<true>(s, vn, bvh, bvl);
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

  // Write this wave's (max, sum, accumulator / vscale) for lanes col < G to
  // the merge slot [G][D + 2]; `hot_layout` selects the coordinate order.
  __device__ __forceinline__ void to_slot(float *slot_base, bool hot_layout) const {
    const float l_wave = sum16_32(l_run);
    if (col < G) {
      float *slot = slot_base + col * (D + 2);
      if (grp == 0) {
        slot[0] = m_run;
        slot[1] = l_wave;
      }
      const float inv = 1.0f / vscale;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int coord = hot_layout ? 16 * q + 4 * grp + r : 8 * (4 * grp + r) + q;
          slot[2 + coord] = accv[q][r] * inv;
        }
      }
    }
  }
};

// Merge kWaves slots [w][G][D + 2] into one (max, sum, accumulator) per head
// element i of [G][D + 2].
__device__ __forceinline__ float merge_waves(const float *slots, int G, int i) {
  const int h = i / (D + 2), j = i % (D + 2);
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, slots[(w * G + h) * (D + 2)]);
  if (M == -INFINITY) return (j == 0) ? -INFINITY : 0.0f;
  if (j == 0) return M;
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = slots[(w * G + h) * (D + 2)];
    if (mw != -INFINITY) v += __builtin_amdgcn_exp2f(mw - M) * slots[(w * G + h) * (D + 2) + j];
  }
  return v;
}

template <int KB>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(const DecodeParams p) {
  using L = Lay<KB>;
  // Static LDS: its base address is a compile-time constant, so table reads
  // fold the table offset into the instruction.
  __shared__ uint32_t lds[L::total];
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (the wave's range of
  // positions, the buffer descriptors) then stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.q_heads / p.kv_heads;
  float *cent = reinterpret_cast<float *>(lds + L::cent);
  float *qw = reinterpret_cast<float *>(lds + L::qwork);
  float *red = reinterpret_cast<float *>(lds + L::red);
  int *flag = reinterpret_cast<int *>(red + 8);
  float *work = reinterpret_cast<float *>(lds);  // merge area after the main loop

  const int nsplit = p.n_cold_splits;
  const int unit = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  const int b = unit / p.kv_heads;
  const int kv = unit % p.kv_heads;
  const long hq0 = static_cast<long>(b) * p.q_heads + static_cast<long>(kv) * G;
  const int s0 = split * p.cold_split_len;
  const int s1 = min(p.cold_len, s0 + p.cold_split_len);
  const int span = max(0, s1 - s0);
  const int per = ((span + kWaves - 1) / kWaves + kChunk - 1) / kChunk * kChunk;
  const int ws = s0 + wave * per;
  const int we = min(s1, ws + per);

  constexpr bool k_packed = KB != 0;
  constexpr int kRowBytes = Wave<KB>::kRowBytes;
  Wave<KB> W;
  W.col = lane & 15;
  W.grp = lane >> 4;
  W.rep4 = (lane & (kRep - 1)) * 4u;
  W.rep4lo = (lane & (L::klo_rep - 1)) * 4u;
  W.lds = lds;
  W.G = G;
  const long rowbase = static_cast<long>(unit) * p.capacity;
  W.kbase = KB ? reinterpret_cast<const char *>(p.k.codes) + rowbase * kRowBytes
               : reinterpret_cast<const char *>(p.k.fp16) + rowbase * kRowBytes;
  W.knbase = KB ? reinterpret_cast<const char *>(p.k.norms + rowbase) : W.kbase;
  W.vbase = reinterpret_cast<const char *>(p.v.codes) + rowbase * 64;
  W.vnbase = reinterpret_cast<const char *>(p.v.norms + rowbase);
  W.koff = static_cast<uint32_t>(W.col * kRowBytes + W.grp * (kRowBytes / 4));
  W.knoff = static_cast<uint32_t>(16 * W.grp);
  W.voff = static_cast<uint32_t>(W.grp * 4 * 64 + W.col * 4);
  W.capacity = p.capacity;
  W.hot_len = p.v.hot > 0 ? p.v.hot : 1;
  W.ring = (p.v.mode == TQ_SIDE_DELEGATED) ? p.v.fp16 + static_cast<long>(unit) * p.v.hot * D : nullptr;
  W.vscale = kVscaleMax;
  W.reset();

  // ---- first chunk in flight while the block builds its tables --------
  ChunkData<KB> A, B;
  if (ws < we) W.load(ws, A);

  for (int i = threadIdx.x; i < kMaxLevels; i += kThreads) {
    cent[i] = p.k_cent[i];
    cent[kMaxLevels + i] = p.v_cent[i];
  }
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const float x = h2f(p.q[hq0 * D + i]);
    qw[i] = k_packed ? x * sign_of(p.sign, i % D) : x;
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
        const float a = qw[h * D + j], c = qw[h * D + j + s];
        qw[h * D + j] = a + c;
        qw[h * D + j + s] = a - c;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  {
    const float qscale = k_packed ? kLog2e / static_cast<float>(D) : kLog2e / sqrtf(static_cast<float>(D));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = 32 * W.grp + 8 * c + 2 * s;
        h[s] = l[s] = 0u;
        if (W.col < G) split_pair(qw[W.col * D + j] * qscale, qw[W.col * D + j + 1] * qscale, h[s], l[s]);
      }
      W.bq[c].hi = as_half8(h[0], h[1], h[2], h[3]);
      W.bq[c].lo = as_half8(l[0], l[1], l[2], l[3]);
    }
  }

  // ---- main loop: chunk t0 is processed while chunk t0 + 32 loads into the
  // other of two register buffers (ping-pong, so nothing is copied) --------
  const long score_row = hq0 + W.col;
  if (ws < we) {
    int t0 = ws;
    for (;;) {
      const bool nb = t0 + kChunk < we;
      if (nb) W.load(t0 + kChunk, B);
      if (t0 + kChunk <= we) {
        W.template cold_chunk<false>(t0, we, A, p.scores, score_row, p.length);
      } else {
        W.template cold_chunk<true>(t0, we, A, p.scores, score_row, p.length);
      }
      t0 += kChunk;
      if (!nb) break;
      const bool na = t0 + kChunk < we;
      if (na) W.load(t0 + kChunk, A);
      if (t0 + kChunk <= we) {
        W.template cold_chunk<false>(t0, we, B, p.scores, score_row, p.length);
      } else {
        W.template cold_chunk<true>(t0, we, B, p.scores, score_row, p.length);
      }
      t0 += kChunk;
      if (!na) break;
    }
  }

  // ---- merge the waves of this block (tables are dead from here on) -----
  __syncthreads();
  W.to_slot(work + wave * G * (D + 2), false);
  __syncthreads();
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + p.ws_part_off);
  float *mypart = part + (static_cast<long>(unit) * nsplit + split) * G * (D + 2);
  for (int i = threadIdx.x; i < G * (D + 2); i += kThreads) store_coherent(mypart + i, merge_waves(work, G, i));

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

  // delegated V: this block also attends over the fp16 hot window
  float *hotp = work + kWaves * G * (D + 2);  // [G][D + 2] merged hot partial
  const int h0 = p.cold_len, h1 = p.length;
  const bool has_hot = h1 > h0;
  if (has_hot) {
    const int hspan = h1 - h0;
    const int hper = ((hspan + kWaves - 1) / kWaves + kChunk - 1) / kChunk * kChunk;
    const int hs = h0 + wave * hper, he = min(h1, hs + hper);
    W.reset();
    W.vscale = 1.0f;
    for (int t0 = hs; t0 < he; t0 += kChunk) {
      W.load(t0, A);
      W.hot_chunk(t0, he, A, p.scores, score_row, p.length);
    }
    W.to_slot(work + wave * G * (D + 2), true);
    __syncthreads();
    for (int i = threadIdx.x; i < G * (D + 2); i += kThreads) hotp[i] = merge_waves(work, G, i);
    __syncthreads();
  }

  // Every load below is independent of the others, so each thread has all of
  // its partial results in flight at once.  Thread (h, j4) owns head h,
  // coordinates 4 j4 .. 4 j4 + 3.
  const float *up = part + static_cast<long>(unit) * nsplit * G * (D + 2);
  float *rot = work;          // [G][D] rotated-domain sum (overwrites the slots)
  float *pln = work + G * D;  // [G][D] plain (hot) sum
  float *Ls = pln + G * D;    // [G] total sums
  float r4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, q4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float Lt = 0.0f;
  int hh = 0, jj = 0;
  const bool mine = threadIdx.x < G * (D / 4);
  if (mine) {
    hh = threadIdx.x / (D / 4);
    jj = 4 * (threadIdx.x % (D / 4));
    float M = -INFINITY;
    for (int sp0 = 0; sp0 < nsplit; sp0 += 16) {
      float mv[16], lv[16], ov[16][4];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int sp = min(sp0 + k, nsplit - 1);
        const float *src = up + (sp * G + hh) * (D + 2);
        mv[k] = (sp0 + k < nsplit) ? load_coherent(src) : -INFINITY;
        lv[k] = load_coherent(src + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[k][e] = load_coherent(src + 2 + jj + e);
      }
      float mg = M;
#pragma unroll
      for (int k = 0; k < 16; ++k) mg = fmaxf(mg, mv[k]);
      if (mg == -INFINITY) continue;
      const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - mg);
      M = mg;
      Lt *= a;
#pragma unroll
      for (int e = 0; e < 4; ++e) r4[e] *= a;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float w = (mv[k] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv[k] - M);
        Lt += w * lv[k];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] += w * ov[k][e];
      }
    }
    if (has_hot) {
      const float mh = hotp[hh * (D + 2)];
      if (mh != -INFINITY) {
        const float mg = fmaxf(M, mh);
        const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - mg);
        const float bh = __builtin_amdgcn_exp2f(mh - mg);
        Lt = Lt * a + bh * hotp[hh * (D + 2) + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r4[e] *= a;
          q4[e] = bh * hotp[hh * (D + 2) + 2 + jj + e];
        }
      }
    }
  }
  __syncthreads();  // hot partial and slots no longer needed
  if (mine) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rot[hh * D + jj + e] = r4[e];
      pln[hh * D + jj + e] = q4[e];
    }
    if (jj == 0) Ls[hh] = Lt;
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

}  // namespace

size_t decode_mfma_lds_bytes(int k_bits, bool share_lut, int G) {
  (void)share_lut;
  switch (k_bits) {
    case 0: return G <= Lay<0>::max_g ? 4 * size_t(Lay<0>::total) : ~size_t(0);
    case 3: return G <= Lay<3>::max_g ? 4 * size_t(Lay<3>::total) : ~size_t(0);
    case 4: return G <= Lay<4>::max_g ? 4 * size_t(Lay<4>::total) : ~size_t(0);
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
  } else if (p.k.mode == TQ_SIDE_PACKED && p.k.bits == 3 && p.v.mode == TQ_SIDE_PACKED) {
    kb = 3;
  } else if (p.k.mode == TQ_SIDE_PACKED && p.k.bits == 4 && p.share_lut && p.v.mode == TQ_SIDE_PACKED) {
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
  if (decode_mfma_lds_bytes(kb, p.share_lut != 0, G) > 65536) return hipErrorInvalidValue;
  const int nsplit = p.n_cold_splits;
  if (nsplit < 1 || nsplit > kMaxSplits || p.n_hot_splits != 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.batch * p.kv_heads * nsplit));
  switch (kb) {
    case 0: hipLaunchKernelGGL(decode_mfma_kernel<0>, grid, dim3(kThreads), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(decode_mfma_kernel<3>, grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
