// Matrix-core quantize-append encoder for packed sides at head_dim 128 and
// 1..4 bits ("TurboQuant KV Cache Quantization in MLX-VLM": "The
// TurboQuantKVCache Class", "How TurboQuant KV Cache Quantization Works").
//
// The rotation of a row is y = H diag(s) x / (n sqrt(d)).  H diag(s) is a
// constant +-1 matrix, and fp16 inputs times +-1 are exact MFMA products, so
// v_mfma_f32_16x16x32_f16 gives H diag(s) x up to the fp32 accumulation; the
// norm only scales the result.  A wave encodes 16 rows per tile:
//
//   A   lane l holds row l % 16, input coordinates 32 q + 8 (l / 16) .. +7 for
//       K-step q: four 16-byte loads straight from the fp16 rows.
//   B   M[j][i] = s_j H[i][j] with column n of N-tile t computing output
//       coordinate i = 8 n + t, so a lane ends up holding 8 consecutive
//       coordinates of its rows.  With j = 32 q + 8 g + s and i = 8 n + t,
//       popcount(i & j) = popcount(n & (4 q + g)) + popcount(t & s): each
//       entry is a per-lane sign times a fixed 8 x 8 Hadamard pattern.  B is
//       built once per block into LDS (16 KB) and read per tile, which keeps
//       the wave at 80 registers: six waves per SIMD on contiguous caches
//       and on paged ones with an append aligned to the tile (general paged
//       appends keep a prefetch buffer: four).
//   D   lane (g = l / 16, n = l % 16) holds rows 4 g + r (r = 0..3),
//       coordinates 8 n .. 8 n + 7, as 8 N-tiles of 4 values.
//
// The norm comes from the same fp16 operands (dot2 instructions, fp32 sums).
// Coding: with a power-of-two scale S, u = y S is exact, and a code table
// over the unit cells [k - S, k - S + 1) holds, per cell, the number of
// scaled thresholds below the cell and the one threshold inside it (the
// host picks S so no cell holds two).  code = base + (u > thr): one table
// read per coordinate, the same decision as counting thresholds below y.
// The 8 codes of a lane pack into 8 b bits; b = 4 is one word per lane, other
// widths assemble words from neighbouring lanes with shuffles.
#include <math.h>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 16;
// cells k = 0 .. 2 S + 2 cover u in [k - S - 1, k - S): one guard cell on
// each side of [-S, S]
constexpr int kLutCells = 2 * kQuantLutMaxScale + 3;

struct LutEntry {
  uint32_t base;  // scaled thresholds below the cell
  float thr;      // the scaled threshold inside the cell, or +inf
};

__device__ __forceinline__ float4_t mma(const half8_t a, const half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8_t as_half8(u32x4_t v) { return __builtin_bit_cast(half8_t, v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, long bytes) {
  const int b = bytes > 0x7fffffffL ? 0x7fffffff : static_cast<int>(bytes > 0 ? bytes : 0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, b, 0x00020000);
}

// Sum over the four 16-lane rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float sum_rows(float x) {
  const u32x2_t a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const u32x2_t b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Build the code table of one side: cells k = 0 .. 2 S + 2 cover u in
// [k - S - 1, k - S).  The guard cells below -S and at or above S hold code 0
// and the top code, so a coordinate a rounding step outside [-1, 1] needs no
// clamp: |y| <= 1 for every row (the rotation is orthonormal), and a non-finite
// u (only from a non-finite row, whose scale is 0) converts to cell 0 of u.
__device__ void build_lut(LutEntry *lut, const float *thr, int bits, float scale) {
  const int S = static_cast<int>(scale);
  const int n_thr = (1 << bits) - 1;
  for (int k = threadIdx.x; k <= 2 * S + 2; k += kThreads) {
    const float lo = static_cast<float>(k - S - 1);
    int cnt = 0;  // thresholds with thr * S < lo (ascending thresholds)
    for (int step = 128; step >= 1; step >>= 1) {
      if (cnt + step <= n_thr && thr[cnt + step - 1] * scale < lo) cnt += step;
    }
    LutEntry e;
    e.base = static_cast<uint32_t>(cnt);
    const float t = cnt < n_thr ? thr[cnt] * scale : INFINITY;
    e.thr = (t < lo + 1.0f) ? t : INFINITY;
    lut[k] = e;
  }
}

// Assemble word n of a row from the 8 b-bit chunks of the row's 16 lanes
// (chunk of lane n covers row bits [8 b n, 8 b n + 8 b)).
template <int BITS>
__device__ __forceinline__ uint32_t row_word(uint32_t chunk, int lane) {
  const int n = lane & 15;
  const int row0 = lane & 48;
  if (BITS == 4) return chunk;
  if (BITS == 2) {
    const uint32_t a = __shfl(chunk, row0 + ((2 * n) & 15));
    const uint32_t b = __shfl(chunk, row0 + ((2 * n + 1) & 15));
    return a | (b << 16);
  }
  if (BITS == 1) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) w |= __shfl(chunk, row0 + ((4 * n + k) & 15)) << (8 * k);
    return w;
  }
  // BITS == 3: word n starts at row bit 32 n = 24 n0 + s0
  const int n0 = (4 * n) / 3;
  const int s0 = 32 * n - 24 * n0;
  const uint32_t a = __shfl(chunk, row0 + (n0 & 15));
  const uint32_t b = __shfl(chunk, row0 + ((n0 + 1) & 15));
  return (a >> s0) | (b << (24 - s0));
}

// floor(x) as an integer in one instruction (v_cvt_flr_i32_f32).
__device__ __forceinline__ int floor_to_int(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// lut0 points at the cell of u = 0 (cell index S + 1 of the side's table).
template <int BITS>
__device__ __forceinline__ void encode_tile(const float4_t (&acc)[8], const float (&inv_s)[4],
                                            const LutEntry *lut0, int lane, uint32_t (&word)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t chunk = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float u = acc[t][r] * inv_s[r];
      const LutEntry e = lut0[floor_to_int(u)];
      const uint32_t c = e.base + (u > e.thr ? 1u : 0u);
      chunk |= c << (BITS * t);
    }
    word[r] = row_word<BITS>(chunk, lane);
  }
}

// PG: paged storage, any append.  Contiguous caches run six waves a SIMD (80
// registers) with no prefetch buffer, the waves hiding each other's load
// latency; the general paged kernel keeps the next tile's operands and
// storage rows in flight (four waves).  AL (with PG false): paged storage
// and an aligned append (offset and n_new multiples of 16), so each tile's
// 16 rows are consecutive positions of one unit inside one block: one table
// entry per tile gives their storage rows, and the tile runs as on a
// contiguous cache.
template <bool PG, bool AL>
__global__ __launch_bounds__(kThreads, PG ? 4 : 6) void quantize_mfma_kernel(const QuantizeParams p, int tiles_k,
                                                                             int tiles_total) {
  __shared__ LutEntry lut[2][kLutCells];
  __shared__ u32x4_t bsh[16][64];  // B operands [4 t + q][lane] for the N-tiles t < 4
  // contiguous stores: each wave's tile of code words (16 rows of up to 16
  // words) and norms, gathered in row order
  __shared__ u32x4_t stage[PG ? 1 : kWaves][68];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;

  if (p.k_lut_scale > 0.0f) build_lut(lut[0], p.k_thr, p.k.bits, p.k_lut_scale);
  if (p.v_lut_scale > 0.0f) build_lut(lut[1], p.v_thr, p.v.bits, p.v_lut_scale);

  // B = diag(s) H^T in the layout described above, for the N-tiles t < 4,
  // written to LDS by wave 0.  Tile t + 4 differs from tile t only by the
  // sign of its k slots 4..7 (popcount((t ^ 4) & s) flips with bit 2 of s),
  // which the product takes from A instead: A with those slots negated.
  if (wave == 0) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t par = static_cast<uint32_t>(__builtin_popcount(n & (4 * q + g)) & 1);
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const int j0 = 32 * q + 8 * g + 2 * pr;  // even: j0 and j0 + 1 share a sign word
      const uint32_t sw = p.sign[j0 >> 5] >> (j0 & 31);
      const uint32_t s0 = (sw & 1u) ^ par, s1 = ((sw >> 1) & 1u) ^ par;
      const uint32_t base = (0x3c00u | (s0 << 15)) | ((0x3c00u | (s1 << 15)) << 16);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t m = (static_cast<uint32_t>(__builtin_popcount(t & (2 * pr)) & 1) << 15) |
                           (static_cast<uint32_t>(__builtin_popcount(t & (2 * pr + 1)) & 1) << 31);
        reinterpret_cast<uint32_t *>(&bsh[4 * t + q][lane])[pr] = base ^ m;
      }
    }
  }
  }
  __syncthreads();  // tables complete

  const long rows = static_cast<long>(p.batch) * p.heads * p.n_new;
  const float rsd = 1.0f / sqrtf(static_cast<float>(D));
  const int stride = gridDim.x * kWaves;
  // A operands of a tile: row n of the tile, coordinates 32 q + 8 g .. + 7.
  // The next tile's operands load while the current one is encoded.
  auto load_tile = [&](int tile, half8_t (&dst)[4]) {
    const int side = tile < tiles_k ? 0 : 1;
    const long r0 = static_cast<long>(side ? tile - tiles_k : tile) * kTileRows;
    const long left = rows - r0;
    const auto rx = rsrc((side ? p.v_new : p.k_new) + r0 * D, (left < kTileRows ? left : kTileRows) * D * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dst[q] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rx, (n * D + 32 * q + 8 * g) * 2, 0, 0));
  };
  // Paged storage: the storage rows of this lane's output rows (4 g + r) of
  // a tile, looked up in the block table together with the tile's loads, so
  // the lookups are in flight while the tile before it is encoded.
  auto paged_rows = [&](int tl, long (&rw)[4]) {
    const int sd_ = tl < tiles_k ? 0 : 1;
    const long q0 = static_cast<long>(sd_ ? tl - tiles_k : tl) * kTileRows;
    const long lf = rows - q0;
    const long b0 = rows <= 0x7fffffffL ? static_cast<long>(static_cast<uint32_t>(q0) / static_cast<uint32_t>(p.n_new))
                                        : q0 / p.n_new;
    const int j0 = static_cast<int>(q0 - b0 * p.n_new);
    // (sequence, head) of the tile's first row and of the next one (a tile
    // crosses at most one boundary), divided once per tile
    const int sq0 = static_cast<int>(b0) / p.heads, hd0 = static_cast<int>(b0) - sq0 * p.heads;
    const int sq1 = hd0 + 1 == p.heads ? sq0 + 1 : sq0, hd1 = hd0 + 1 == p.heads ? 0 : hd0 + 1;
    // the lane's four rows are consecutive positions of one unit unless they
    // cross the unit boundary, a block boundary or the end of the rows: the
    // first row is looked up, the others follow it; only lanes with such a
    // crossing look each row up
    const int trf = min(4 * g, static_cast<int>(lf) - 1);
    const bool wrapf = j0 + trf >= p.n_new;
    const unsigned tf = static_cast<unsigned>(p.offset + j0 + trf - (wrapf ? p.n_new : 0));
    const unsigned ubs = static_cast<unsigned>(p.pg.bs), blkf = tf / ubs;
    const int within = static_cast<int>(tf - blkf * ubs);
    const int sqf = wrapf ? sq1 : sq0, hdf = wrapf ? hd1 : hd0;
    // (-1: a block outside the pools, whose rows are not written)
    const long ef = valid_block(p.pg, p.pg.table[sqf * p.pg.max_blocks + static_cast<int>(blkf)]);
    rw[0] = ef < 0 ? -1L : (ef * p.pg.kv_heads + hdf) * p.pg.bs + within;
    const bool run = 4 * g + 3 <= lf - 1 && (j0 + 4 * g + 3 >= p.n_new) == wrapf && within + 3 < p.pg.bs;
    if (run) {
#pragma unroll
      for (int r = 1; r < 4; ++r) rw[r] = ef < 0 ? -1L : rw[0] + r;
    } else {
#pragma unroll
      for (int r = 1; r < 4; ++r) {
        const int tr = min(4 * g + r, static_cast<int>(lf) - 1);
        const bool wrap = j0 + tr >= p.n_new;
        rw[r] = paged_row(p.pg, wrap ? sq1 : sq0, wrap ? hd1 : hd0, p.offset + j0 + tr - (wrap ? p.n_new : 0));
      }
    }
  };
  // encode tile `tile` from its A operands (and, paged, its storage rows)
  // AL: the storage row of the tile's first row (-1: a block outside the
  // pools, whose rows are not written).  The table entry is read with a
  // vector load issued after the tile's operands, so waiting for the
  // operands does not wait for it.
  auto aligned_row = [&](int tl) -> long {
    const int sd_ = tl < tiles_k ? 0 : 1;
    const unsigned q0 = static_cast<unsigned>(sd_ ? tl - tiles_k : tl) * kTileRows;
    const unsigned un = static_cast<unsigned>(p.n_new), uh = static_cast<unsigned>(p.heads);
    const unsigned bh = q0 / un, i0 = q0 - bh * un;
    const unsigned b = bh / uh, kv = bh - b * uh;
    const unsigned t = static_cast<unsigned>(p.offset) + i0, ubs = static_cast<unsigned>(p.pg.bs);
    const unsigned blk = t / ubs;
    const auto rt = rsrc(p.pg.table + static_cast<long>(b) * p.pg.max_blocks, 4L * p.pg.max_blocks);
    const int entry = __builtin_amdgcn_readfirstlane(
        static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rt, 4 * blk, 0, 0)));
    const long e = valid_block(p.pg, entry);
    return e < 0 ? -1L : (e * p.pg.kv_heads + kv) * p.pg.bs + static_cast<long>(t - blk * ubs);
  };
  auto encode = [&](int tile, const half8_t (&a)[4], const long (&prow)[4], long al_row) {
      const int side = tile < tiles_k ? 0 : 1;
      const SideDev &sd = side ? p.v : p.k;
      const float scale = side ? p.v_lut_scale : p.k_lut_scale;
      const long r0 = static_cast<long>(side ? tile - tiles_k : tile) * kTileRows;
      // rows of this tile that exist (the last tile may be short)
      const int left = rows - r0 < kTileRows ? static_cast<int>(rows - r0) : kTileRows;

      // squared norm of row n: fp16 products are exact, sums in fp32
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const half2_t h = {a[q][e], a[q][e + 1]};
          ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        }
      }
      ss = sum_rows(ss);

      float4_t acc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      asm volatile("" ::: "memory");  // B is read from LDS per tile, not kept in registers
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4_t af = __builtin_bit_cast(u32x4_t, a[q]);
        af[2] ^= 0x80008000u;
        af[3] ^= 0x80008000u;
        const half8_t a_flip = as_half8(af);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4_t b = bsh[4 * t + q][lane];
          acc[t] = mma(a[q], as_half8(b), acc[t]);
          acc[t + 4] = mma(a_flip, as_half8(b), acc[t + 4]);
        }
      }

      // rows 4 g + r of this lane: norm and 1 / (n sqrt(d)) times the table
      // scale (a power of two, so the scaling is exact)
      float nrm[4], inv_s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s2 = __shfl(ss, 4 * g + r);
        nrm[r] = __builtin_amdgcn_sqrtf(s2);  // v_sqrt_f32: within 1 ulp
        inv_s[r] = nrm[r] > 0.0f ? scale * (rsd * __builtin_amdgcn_rcpf(nrm[r])) : 0.0f;
      }

      uint32_t word[4];
      const LutEntry *lut0 = lut[side] + static_cast<int>(scale) + 1;
      switch (sd.bits) {
        case 1: encode_tile<1>(acc, inv_s, lut0, lane, word); break;
        case 2: encode_tile<2>(acc, inv_s, lut0, lane, word); break;
        case 3: encode_tile<3>(acc, inv_s, lut0, lane, word); break;
        default: encode_tile<4>(acc, inv_s, lut0, lane, word); break;
      }

      // output rows: tile row tr = 4 g + r is input row r0 + tr = (bh, i).
      // n_new >= 16, so the tile crosses at most one (batch, head) boundary;
      // crossing it skips the capacity - n_new rows the append leaves alone.
      // (32-bit division when the rows allow: a 64-bit one costs about a
      // hundred scalar instructions per tile)
      const long bh0 = rows <= 0x7fffffffL ? static_cast<long>(static_cast<uint32_t>(r0) / static_cast<uint32_t>(p.n_new))
                                           : r0 / p.n_new;
      const int i0 = static_cast<int>(r0 - bh0 * p.n_new);
      const int W = sd.words;
      // AL: the tile's rows start at al_row and never cross a unit
      if (AL && al_row < 0) return;
      const long row0 = AL ? al_row : bh0 * p.capacity + p.offset + i0;
      uint32_t *codes0 = sd.codes + row0 * W;
      float *norms0 = sd.norms + row0;
      const int skip = p.capacity - p.n_new;
      if (PG) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (4 * g + r >= left || prow[r] < 0) continue;
          if (n < W) sd.codes[prow[r] * W + n] = word[r];
          if (n == r) sd.norms[prow[r]] = nrm[r];
        }
        return;
      }
      // (AL: always; n_new is a multiple of 16 there)
      if (AL || (left == kTileRows && i0 + kTileRows <= p.n_new)) {
        // the tile's 16 rows are consecutive storage rows: gather them in
        // row order in LDS, then write the 16 W words with one 16-byte
        // store per lane (16 W is a multiple of 4: W = 4 bits) and the 16
        // norms with one word store per lane
        uint32_t *st = reinterpret_cast<uint32_t *>(&stage[PG ? 0 : wave][0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n < W) st[(4 * g + r) * W + n] = word[r];
          if (n == r) st[256 + 4 * g + r] = __float_as_uint(nrm[r]);
        }
        __builtin_amdgcn_wave_barrier();
        // the lane index recomputed here: offsets derived from the kernel's
        // copy would be kept in registers across the whole loop
        uint32_t lid;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
        if (4 * lid < static_cast<uint32_t>(kTileRows * W))
          *reinterpret_cast<u32x4_t *>(codes0 + 4 * lid) = *reinterpret_cast<const u32x4_t *>(st + 4 * lid);
        if (lid < kTileRows) norms0[lid] = __uint_as_float(st[256 + lid]);
        __builtin_amdgcn_wave_barrier();  // the stage is read before the next tile writes it
        return;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 4 * g + r;
        if (tr >= left) continue;
        const int rel = tr + (i0 + tr >= p.n_new ? skip : 0);
        if (n < W) codes0[rel * W + n] = word[r];
        if (n == r) norms0[rel] = nrm[r];
      }
  };
  int tile = blockIdx.x * kWaves + wave;
  if (PG) {
    half8_t a[4], an[4];
    long prow[4], prow_n[4];
    if (tile < tiles_total) {
      load_tile(tile, an);
      paged_rows(tile, prow_n);
    }
    for (; tile < tiles_total; tile += stride) {
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = an[q];
#pragma unroll
      for (int r = 0; r < 4; ++r) prow[r] = prow_n[r];
      if (tile + stride < tiles_total) {
        load_tile(tile + stride, an);
        paged_rows(tile + stride, prow_n);
      }
      encode(tile, a, prow, 0L);
    }
  } else {
    const long none[4] = {0, 0, 0, 0};
    for (; tile < tiles_total; tile += stride) {
      half8_t a[4];
      load_tile(tile, a);
      encode(tile, a, none, AL ? aligned_row(tile) : 0L);
    }
  }
}

}  // namespace

float quantize_lut_scale(const float *thr, int bits) {
  const int n_thr = (1 << bits) - 1;
  double gap = 2.0;
  for (int k = 0; k + 1 < n_thr; ++k) {
    const double d = static_cast<double>(thr[k + 1]) - static_cast<double>(thr[k]);
    if (d < gap) gap = d;
  }
  for (int s = 1; s <= kQuantLutMaxScale; s *= 2) {
    // consecutive scaled thresholds more than one cell apart: a unit cell
    // never holds two
    if (gap * s > 1.0) return static_cast<float>(s);
  }
  return 0.0f;
}

hipError_t launch_quantize_mfma(const QuantizeParams &p, hipStream_t stream) {
  if (p.head_dim != D || p.n_new < kTileRows) return hipErrorInvalidValue;
  const long rows = static_cast<long>(p.batch) * p.heads * p.n_new;
  const long tiles_side = (rows + kTileRows - 1) / kTileRows;
  const bool k_on = p.k_lut_scale > 0.0f, v_on = p.v_lut_scale > 0.0f;
  for (int side = 0; side < 2; ++side) {
    const SideDev &s = side ? p.v : p.k;
    const float sc = side ? p.v_lut_scale : p.k_lut_scale;
    if (sc > 0.0f && (s.mode != TQ_SIDE_PACKED || s.bits < 1 || s.bits > 4 ||
                      sc > static_cast<float>(kQuantLutMaxScale) || s.words != 4 * s.bits))
      return hipErrorInvalidValue;
  }
  const long tiles_k = k_on ? tiles_side : 0;
  const long tiles_total = tiles_k + (v_on ? tiles_side : 0);
  if (tiles_total == 0) return hipSuccess;
  if (tiles_total > 0x7fffffffL) return hipErrorInvalidValue;
  // a paged append whose offset and length are multiples of the tile keeps
  // every tile inside one block (blocks are multiples of 32 positions)
  // (and its row indices fit the aligned path's 32-bit arithmetic)
  const bool aligned = p.pg.table && p.offset % kTileRows == 0 && p.n_new % kTileRows == 0 &&
                       p.pg.bs % kTileRows == 0 && rows <= 0x7fffffffL;
  const bool general = p.pg.table && !aligned;
  // up to one round at the kernel's occupancy: six (general paged: four)
  // blocks per CU
  const long cap = general ? 1024 : 1536;
  const long blocks = std::min<long>((tiles_total + kWaves - 1) / kWaves, cap);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if (general) {
    hipLaunchKernelGGL((quantize_mfma_kernel<true, false>), grid, block, 0, stream, p, static_cast<int>(tiles_k),
                       static_cast<int>(tiles_total));
  } else if (aligned) {
    hipLaunchKernelGGL((quantize_mfma_kernel<false, true>), grid, block, 0, stream, p, static_cast<int>(tiles_k),
                       static_cast<int>(tiles_total));
  } else {
    hipLaunchKernelGGL((quantize_mfma_kernel<false, false>), grid, block, 0, stream, p, static_cast<int>(tiles_k),
                       static_cast<int>(tiles_total));
  }
  return hipGetLastError();
}

}  // namespace tq
