// Split-context decode attention from the packed cache on the matrix cores
// ("TurboQuant KV Cache Quantization in MLX-VLM", "How TurboQuant KV Cache
// Quantization Works": scores straight from the compressed representation;
// FAQ on dequantization: one stored rotation plus codebooks; mlxcel
// "TurboQuant KV cache", "Available modes": fp16 K with TurboQuant V and the
// delegated hot/cold V split).
//
// head_dim 128, V codes of 2 to 4 bits, K packed (2 to 4 bits) or fp16, up
// to 8 query heads per KV head (and INT8 on both sides).  Grid = (B * Hkv units) x splits, about one block per
// compute unit (12 waves for packed K, 8 for fp16 K).  A block issues its first
// loads, builds its lookup tables and rotated query while they are in
// flight, then each wave walks its share of the split in chunks of 32
// positions, loading chunk i + 1 while it computes chunk i:
//
//   score   v_mfma_f32_16x16x32_f16 with M = 16 positions, N = 16 (hi and
//           lo halves of the G query heads, rest padding), K = 32
//           coordinates.  A holds the centroids of the position's codes,
//           decoded two codes at a time from pair tables in LDS (32 replicas
//           of every 32-bit entry, one per bank, so any index pattern reads
//           without bank conflicts); B holds R q, rotated once per block with
//           1/sqrt(d) and log2(e) folded in.  Times the position's norm this
//           is the base-2 logit.
//   softmax online per query head; the accumulators are only rescaled when
//           the running maximum grows by more than 2^8.
//   value   the same MFMA with M = 16 (the hi and lo weights of the G
//           heads, rest padding), N = 16 coordinates, K = 32 positions.  A
//           holds p_i n_i times a power of two that keeps fp16 in range
//           (lowered lazily when a larger norm arrives).  Each lane loads the
//           codes of 8 coordinates of 8 positions and pairs the codes of two
//           positions at one coordinate in registers, so B (one coordinate
//           of 8 positions a lane) comes from pair-table reads.  The sum
//           stays in the rotated domain.
//   precision  fp16 operands carry 11 bits, and the output of a diffuse
//           softmax is much smaller than the rows it averages, so plain fp16
//           leaves output errors near 1e-3.  Each fp16 operand that is not
//           exact is therefore a hi + lo pair (lo = the fp16 rounding of the
//           remainder): the score takes (A_hi + A_lo)(B_hi + B_lo) in two
//           MFMAs, B_hi and B_lo side by side in N; the value sum takes
//           A_hi (P_hi + P_lo); fp16 K rows are exact (one MFMA).
//
// The waves merge in LDS (one slot each) and the block writes one partial
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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;
// KB selects the K storage: 2, 3 or 4 (packed codes, rotated domain), 0
// (fp16 rows), kInt8 (INT8 absmax: one signed byte a coordinate and a float
// scale a row, on both sides; original domain, no codebook).
constexpr int kInt8 = 8;
template <int KB>
constexpr bool rotated_k() { return KB == 2 || KB == 3 || KB == 4; }
// VB selects the packed V storage: 2, 3 or 4 bits a code (kInt8 with INT8
// K: INT8 bytes).  V bytes a row:
template <int VB>
constexpr int v_row_bytes() { return D * VB / 8; }
// Waves per block: 12 for packed K (about 160 registers a lane, so three
// waves a SIMD), 8 for fp16 K rows and for INT8 (about 200-250 registers,
// two a SIMD).  One block per compute unit either way.
template <int KB>
constexpr int waves_of() { return (KB == 0 || KB == kInt8) ? 8 : 12; }
constexpr int kMaxWaves = 12;
constexpr int kChunk = kMfmaChunk;
constexpr int kRep = 32;          // pair-table replicas, one per LDS bank
constexpr int kMaxSplits = kMfmaMaxSplits;  // splits per unit (bounded by the host)
constexpr float kRescale = 8.0f;  // lazy rescaling threshold (log2 units)
constexpr float kVscaleMax = 1099511627776.0f;  // 2^40: start and ceiling of the V scale

// Static LDS layout (32-bit words).  The lookup tables hold fp16 pairs for a
// code pair index e (first code in the low bits, its centroid in the low
// half).  Entry e occupies 256 bytes at byte e * 256: 32 replicas of the
// entry at +4 r (lane r of each 32-lane half reads its own bank, so any index
// pattern reads without bank conflicts) and 32 replicas of a second table at
// +128 + 4 r.  A byte address is then (e << 8) | 4 r, which one v_perm_b32
// builds from a byte-aligned pair index.
//   KB = 0, 4   V hi in the first half of entries 0..255; for KB = 4 K lo in
//               the second half (K hi is the V table: one 4-bit codebook)
//   KB = 3      K hi / K lo in the first / second half of entries 0..255,
//               indexed by a byte whose low 6 bits hold a pair of 3-bit codes
//               (the top 2 bits are ignored, so every pair is read straight
//               from a byte of the code stream shifted by 0, 6, 12, ...);
//               V hi in the first half of entries 256..511
//   KB = 4, VB = 3   as KB = 3, with 4-bit K pairs (a whole byte)
//   KB = 2      as KB = 3, indexed by a byte whose low 4 bits hold a pair of
//               2-bit codes (the top 4 bits ignored: nibble n of a word is
//               byte n / 2 of the word, or of the word shifted right by 4)
// 3- and 2-bit V tables are indexed the same way: the low 6 or 4 bits hold
// the codes of two positions at one coordinate, the rest is ignored.
// After the main loop the table area is reused for the merges.
constexpr int kTableWords = 256 * 64;  // one 256-entry region (64 KB)
// K hi / K lo in the first region and V in the second whenever K's pairs
// need tables of their own: 2- and 3-bit K, and 4-bit K beside 3-bit V
template <int KB, int VB>
constexpr bool two_tables() { return KB == 2 || KB == 3 || (KB == 4 && VB == 3); }
template <int KB, int VB>
constexpr int table_words() { return two_tables<KB, VB>() ? 2 * kTableWords : kTableWords; }
template <int KB, int VB>
constexpr uint32_t v_table_byte() { return two_tables<KB, VB>() ? 4u * kTableWords : 0u; }
// A partial result (merge slot, workspace partial) of one query head: max,
// sum, two pad words, then the D accumulator values, so the values start
// 16-byte aligned.
constexpr int kPS = D + 4;
constexpr int kPV = 4;
constexpr int kKloOff = 128;  // byte offset of the K lo table from the K hi / V one

template <int KB, int VB, int GP>
struct Lay {
  static constexpr int qstride = D + 4;                  // padded row: fewer bank conflicts
  static constexpr int qwork = table_words<KB, VB>();    // [GP][D + 4] rotated query
  static constexpr int red = qwork + GP * qstride;     // flag
  static constexpr int prog = red + 4;                 // [kMaxWaves] chunks done per wave
  static constexpr int qinv = red + 16;                // [8] per head: the score's query scale
  static constexpr int bmax = red + 24;                // sparse-V: [8 heads][16 waves] exchanged maxima;
                                                       // fused append (exact decode): [32] code bytes of one row
  static constexpr int tail = red + 152;
  // Merge slots of the main loop's waves: an area of their own when it fits
  // (a wave then writes its slot as soon as its own loop ends), else over
  // the tables once every wave is done with them.
  static constexpr int kLdsWords = 160 * 1024 / 4;
  static constexpr bool own_slots = tail + kMaxWaves * GP * kPS <= kLdsWords;
  static constexpr int slots = own_slots ? tail : 0;
  static constexpr int total = own_slots ? tail + kMaxWaves * GP * kPS : tail;
  static_assert((kMaxWaves + 1) * GP * kPS <= kTableWords, "merges must fit in the table area");
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

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Two signed bytes of an INT8 K row as an exact fp16 pair.  w holds four
// bytes already offset by 128 (x ^ 0x80 = x + 128 as an unsigned byte);
// bytes B and B + 1 are placed under the exponent byte 0x64, which reads as
// 1024 + (x + 128), and 1152 is subtracted (exact: every value involved is
// an integer below 2048).
template <int B>
__device__ __forceinline__ uint32_t i8_pair_exact(uint32_t w) {
  const uint32_t e = __builtin_amdgcn_perm(0x64646464u, w, 0x04000400u | ((B + 1) << 16) | B);
  const half2_t h = __builtin_bit_cast(half2_t, e) - half2_t{1152.0f16, 1152.0f16};
  return __builtin_bit_cast(uint32_t, h);
}

// One byte from each of two INT8 V rows (byte B of a and of b, both offset
// by 128) as an fp16 pair x_a 2^-10, x_b 2^-10: the byte as the low bits of
// an fp16 is the subnormal (x + 128) 2^-24; times 2^14 minus 2^-3 is x 2^-10
// exactly (one packed fused multiply-add; fp16 subnormals are kept).
template <int B>
__device__ __forceinline__ uint32_t i8_cross_pair(uint32_t a, uint32_t b) {
  const uint32_t e = __builtin_amdgcn_perm(b, a, 0x0c000c00u | ((4 + B) << 16) | B);
  const half2_t h = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, e), half2_t{16384.0f16, 16384.0f16},
                                              half2_t{-0.125f16, -0.125f16});
  return __builtin_bit_cast(uint32_t, h);
}

// LDS word at byte address `addr` plus a compile-time byte offset.
template <int OFF>
__device__ __forceinline__ uint32_t lds_at(const uint32_t *lds, uint32_t addr) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lds) + addr + OFF);
}

// Same, as a read the compiler may not merge with a neighbouring one into a
// two-address instruction: merging a hi and a lo table read of one address
// lands the two halves in adjacent registers, while the MFMA operands want
// four hi and four lo words each in consecutive registers (the merge then
// costs register copies).
template <int OFF>
__device__ __forceinline__ uint32_t lds_at_sep(const uint32_t *lds, uint32_t addr) {
  typedef __attribute__((address_space(3))) const volatile uint32_t lds_u32;
  return *reinterpret_cast<lds_u32 *>(addr + OFF);
}

// Smallest power of two >= x (x > 0), as a float; 1 for x <= 0.
__device__ __forceinline__ float pow2_ceil(float x) {
  if (!(x > 0.0f)) return 1.0f;
  int e;
  const float m = frexpf(x, &e);  // x = m 2^e, m in [0.5, 1)
  return ldexpf(1.0f, m == 0.5f ? e - 1 : e);
}

// Cache policy of a buffer load that reads past the non-coherent caches
// (sc1), the same bits an agent-scope atomic load carries.
constexpr int kCoherentLoad = 16;

// Buffer resource over [base, base + bytes): loads past the end read 0.
constexpr int kBufFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes > 0 ? bytes : 0, kBufFlags);
}

__device__ __forceinline__ float4 bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, int imm) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + imm, 0, 0);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// Byte address (e << 8) | rep4 of table entry e = byte K of w.
template <int K>
__device__ __forceinline__ uint32_t baddr(uint32_t w, uint32_t rep4) {
  return __builtin_amdgcn_perm(w, rep4, 0x0c0c0000u | ((4u + K) << 8));
}

// The same for a table in the second 64 KB: rep4v = 4 r + 65536, and byte 2
// of the address is taken from it.
template <int K>
__device__ __forceinline__ uint32_t baddr_hi(uint32_t w, uint32_t rep4v) {
  return __builtin_amdgcn_perm(w, rep4v, 0x0c020000u | ((4u + K) << 8));
}

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }

// DPP controls (row = 16 lanes, bank = 4 lanes of a row).
constexpr int kRowShl = 0x100, kRowShr = 0x110, kRowRor = 0x120;

template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xf, BANKS, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t src) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(src), CTRL, 0xf, 0xf, true));
}
// DPP move into the lanes of the banks in BANKS; other lanes keep `old`.
// kRowShl + 0 is the identity (row_shl:0 encodes quad_perm [0,1,2,3]).
template <int CTRL, int BANKS>
__device__ __forceinline__ uint32_t dpp_bank(uint32_t old, uint32_t src) {
  constexpr int ctrl = CTRL == 0x100 ? 0xe4 : CTRL;
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(src), ctrl, 0xf, BANKS, false));
}

// Reductions over the 64 / GP lanes of one query head in the compact layout
// (lanes whose column agrees modulo GP).
template <int GP>
__device__ __forceinline__ float head_max(float x) {
  if (GP == 4) x = fmaxf(x, dpp_f<kRowRor + 4, 0xf>(0.0f, x));
  x = fmaxf(x, dpp_f<kRowRor + 8, 0xf>(0.0f, x));
  const u32x2_t a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const u32x2_t b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
template <int GP>
__device__ __forceinline__ float head_sum(float x) {
  if (GP == 4) x += dpp_f<kRowRor + 4, 0xf>(0.0f, x);
  x += dpp_f<kRowRor + 8, 0xf>(0.0f, x);
  const u32x2_t a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const u32x2_t b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One Walsh-Hadamard butterfly at lane stride M (lane l pairs with l ^ M):
// the lower lane gets x + partner, the upper partner - x.  Strides below 16
// move data with DPP, 16 and 32 with the lane-swap instructions.
template <int M>
__device__ __forceinline__ float xor_butterfly(float x, int lane) {
  const bool upper = (lane & M) != 0;
  if (M == 16 || M == 32) {
    const u32x2_t ab = (M == 16) ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                                 : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float a = __uint_as_float(ab[0]), b = __uint_as_float(ab[1]);  // lower, upper lane's value
    return upper ? a - b : a + b;
  }
  float pt;
  if (M == 1) {
    pt = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
  } else if (M == 2) {
    pt = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
  } else {
    // banks with bit M clear read lane + M, the others lane - M
    constexpr int lo_banks = M == 4 ? 0x5 : 0x3;
    pt = dpp_f<kRowShl + M, lo_banks>(0.0f, x);
    pt = dpp_f<kRowShr + M, 0xf ^ lo_banks>(pt, x);
  }
  return upper ? pt - x : x + pt;
}

// Fused append: the new position of one unit written at storage row `row`
// of one side as the encoder writes it ("TurboQuant KV Cache Quantization in
// MLX-VLM", "How TurboQuant KV Cache Quantization Works"): an fp16 row is
// copied; an INT8 row coded by its absmax; a packed row is normalised,
// rotated by diag(s) then H, scaled by
// 1 / (n sqrt(d)), coded as the number of thresholds below each coordinate
// and packed LSB-first.  One wave: lane l holds coordinates l and l + 64.
// `stage` is 32 words of this wave's LDS for the codes (a byte per
// coordinate).  A row in an out-of-range block (row < 0) takes no writes.
// x0, x1: the fp16 bits of coordinates lane and lane + 64 of the new row.
// The thresholds and sign words are read with uniform indices only (scalar
// loads of the kernel arguments): a per-lane index would make each step of
// a search a memory round trip.
__device__ __forceinline__ void append_side(const SideDev &s, const float (&thr)[16],
                                            const uint32_t (&sign)[kMaxSignWords], uint16_t x0, uint16_t x1,
                                            long row, int lane, uint32_t *stage) {
  if (row < 0) return;
  if (s.mode == TQ_SIDE_FP16) {
    s.fp16[row * D + lane] = x0;
    s.fp16[row * D + lane + 64] = x1;
    return;
  }
  float a = h2f(x0), c = h2f(x1);
  if (s.mode == TQ_SIDE_INT8) {
    // absmax: one signed byte a coordinate (byte j of the row), the scale
    // max |x| / 127 in the norm slot
    float m = fmaxf(fabsf(a), fabsf(c));
    for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
    uint8_t *b8 = reinterpret_cast<uint8_t *>(s.codes + row * s.words);
    b8[lane] = static_cast<uint8_t>(m > 0.0f ? int8_code(a, m) : 0);
    b8[lane + 64] = static_cast<uint8_t>(m > 0.0f ? int8_code(c, m) : 0);
    if (lane == 0) s.norms[row] = m / 127.0f;
    return;
  }
  float ss = a * a + c * c;
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float n = sqrtf(ss);
  const float inv = (n > 0.0f) ? 1.0f / (n * sqrtf(static_cast<float>(D))) : 0.0f;
  const uint32_t sa = lane < 32 ? sign[0] : sign[1], sb = lane < 32 ? sign[2] : sign[3];
  a = ((sa >> (lane & 31)) & 1u) ? -a : a;
  c = ((sb >> (lane & 31)) & 1u) ? -c : c;
  float y0 = a + c, y1 = a - c;
  y0 = xor_butterfly<32>(y0, lane);
  y1 = xor_butterfly<32>(y1, lane);
  y0 = xor_butterfly<16>(y0, lane);
  y1 = xor_butterfly<16>(y1, lane);
  y0 = xor_butterfly<8>(y0, lane);
  y1 = xor_butterfly<8>(y1, lane);
  y0 = xor_butterfly<4>(y0, lane);
  y1 = xor_butterfly<4>(y1, lane);
  y0 = xor_butterfly<2>(y0, lane);
  y1 = xor_butterfly<2>(y1, lane);
  y0 = xor_butterfly<1>(y0, lane);
  y1 = xor_butterfly<1>(y1, lane);
  // code: the number of thresholds below the coordinate (ascending
  // thresholds, 2^bits - 1 of them; at most 4 bits here)
  const float u0 = y0 * inv, u1 = y1 * inv;
  const int nt = (1 << s.bits) - 1;
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    if (k < nt) {
      c0 += u0 > thr[k] ? 1 : 0;
      c1 += u1 > thr[k] ? 1 : 0;
    }
  }
  uint8_t *st8 = reinterpret_cast<uint8_t *>(stage);
  st8[lane] = static_cast<uint8_t>(c0);
  st8[lane + 64] = static_cast<uint8_t>(c1);
  // the stage is this wave's own: its LDS accesses complete in order, so
  // only the compiler has to keep the reads after the writes
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  // word w holds bits 32 w .. 32 w + 31 of the stream, code j at bit b j
  if (lane < s.words) {
    const int b = s.bits;
    const int j0 = 32 * lane / b, j1 = min((32 * lane + 31) / b, D - 1);
    uint64_t acc = 0;
    for (int j = j0; j <= j1; ++j) acc |= static_cast<uint64_t>(st8[j]) << (b * j - 32 * lane + 32);
    s.codes[row * s.words + lane] = static_cast<uint32_t>(acc >> 32);
  }
  if (lane == 0) s.norms[row] = n;
}

// Global-memory data of one chunk of 32 positions for one lane.
template <int KB, int VB, int GP>
struct ChunkData {
  static constexpr int kw = KB == 0 ? 16 : (KB == kInt8 ? 8 : KB);  // K dwords per M-tile
  static constexpr int kvw = (VB == 4 || VB == 2) ? 8 : 16;    // V dwords
  static constexpr int nv = GP / 2;                            // compact values per lane
  uint32_t k[2][kw];   // K words (packed), fp16 or INT8 row piece, M-tiles 0 and 1
  float kn[nv];        // K norms (INT8: scales) of the lane's compact positions
  uint32_t v[kvw];     // V: code word `col` (2-bit: the dword holding the 16 bits
                       // of coordinates 8 col .. 8 col + 7; 3-bit: the two dwords
                       // holding their 24 bits; INT8: bytes 8 col .. 8 col + 7)
                       // of the 8 positions of this lane group
  float vn[nv];        // V norms (INT8: scales) of the compact positions
  bool vskip;          // sparse-V: the V codes were not loaded (predicted skippable)
};

// Lane roles.  MFMA layouts (v_mfma_f32_16x16x32_f16): A lane l holds row
// l % 16, k = 8 (l / 16) + s; B lane l holds k = 8 (l / 16) + s, column
// l % 16; D lane l holds rows 4 (l / 16) + r, column l % 16.  With col =
// l % 16 and grp = l / 16, position slot s8 (0..7) of lane group grp is chunk
// position 16 (s8 / 4) + 4 grp + s8 % 4; the score D of M-tile m, row r is
// slot 4 m + r.  Only GP of the 16 head columns are real, so the softmax runs
// on a compact layout: lane (grp, col = GP kc + h) holds head h at slots
// nv kc .. nv kc + nv - 1 (nv = GP / 2 consecutive positions), moved there
// from lane (grp, h) with DPP row shifts, and moved back the same way for the
// value MFMA's B operand.
template <int KB, int VB, int GP, bool PG>
struct Wave {
  static constexpr int NV = GP / 2;
  static constexpr int kRowBytes = KB == 0 ? 2 * D : (KB == kInt8 ? D : D * KB / 8);
  static constexpr int kVRow = v_row_bytes<VB>();
  // per-lane constants
  int col, grp, cpos;   // cpos: chunk position of the lane's first compact slot
  uint32_t rep4;        // 4 r: the lane's replica
  uint32_t rep4v;       // 4 r + the V table's byte offset
  uint32_t koff, knoff, voff;   // lane byte offsets inside a chunk
  uint32_t vsh;         // 3-bit V: bit offset of the lane's 24 bits in its first
                        // dword; 2-bit V: v_perm selector of its 16 bits
  bool vlast;           // 3-bit V: lane column 15, whose bits all lie in its second dword
  const uint32_t *lds;
  uint32_t bmax_at;     // sparse-V: LDS byte address of the exchanged maxima [8 heads][16 waves]
  int wave_id;
  half8_t bq[4];         // R q: column h < GP hi, column GP + h lo of head h
  // per-unit bases
  const char *kbase;   // K codes or fp16 rows of this unit
  const char *knbase;  // K norms
  const char *vbase;   // V codes
  const char *vnbase;  // V norms
  const uint16_t *ring;
  int capacity, hot_len, G;
  Paging pg;           // PG: where the unit's rows live
  int unit;
  float sparse_lg;     // sparse-V threshold (log2), -inf = exact
  float block_ref;     // sparse-V: the largest running maximum of the lane's head
                       // the block's waves had after their first chunk (-inf: none)
  bool pred_skip;      // sparse-V: the wave's last chunk was skippable, so the
                       // next chunk's V codes are not loaded up front
  float qinv;          // the lane's head (compact layout): the power of two
                       // that undoes the query's scaling in B (see the prologue)
  float chunk_max;     // the last softmax's chunk maximum of the lane's head
  float vscale;        // per head (compact layout, the lane's head): a power
                       // of two keeping the value weights p n vscale in fp16's
                       // range (see softmax)
  // running state (compact layout: head col % GP)
  float m_run, l_run;
  float4_t accv[8];    // D layout: head col, coordinates of tile q

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) accv[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // First storage row of the chunk at t0.  Paged: t0 is a multiple of 32
  // and a block a multiple of 32 positions, so the chunk's rows are
  // consecutive rows of one block; -1 when the block lies outside the pools.
  // (A wave past the end of its split may ask for t0 >= capacity: it reads
  // nothing, and the table is not read.)
  __device__ __forceinline__ long row_of(int t0) const {
    if (!PG) return t0;
    return t0 < capacity ? cache_row(pg, unit, t0, capacity) : 0L;
  }

  // Paged: the table entry of the chunk at t0 as a vector load (its wait is
  // ordered with the chunk loads, unlike a scalar load's, which every LDS
  // wait would have to include); past the table it reads 0.
  __device__ __forceinline__ uint32_t blk_fetch(int t0) const {
    if (!PG) return 0u;
    const int b = unit / pg.kv_heads;
    const auto rt = rsrc(pg.table + static_cast<long>(b) * pg.max_blocks, 4 * pg.max_blocks);
    return __builtin_amdgcn_raw_buffer_load_b32(rt, 4 * (t0 / pg.bs), 0, 0);
  }
  __device__ __forceinline__ long row_from(uint32_t blk, int t0) const {
    if (!PG) return t0;
    const int kv = unit % pg.kv_heads;
    const long bl = valid_block(pg, static_cast<int>(__builtin_amdgcn_readfirstlane(blk)));
    return bl < 0 ? -1L : (bl * pg.kv_heads + kv) * pg.bs + t0 % pg.bs;
  }

  __device__ __forceinline__ void load(int t0, ChunkData<KB, VB, GP> &c) const { load_row(row_of(t0), t0, c); }

  // rows [t0, t0 + 32) at most, from storage row row0 on; rows past the
  // unit's capacity, and every row of an out-of-range block (row0 = -1),
  // read 0
  // vskip (sparse-V): the V codes go through an empty buffer resource, which
  // reads nothing and returns zeros (the same loads are issued, so the
  // wave's waits stay static); the chunk notes it, and reloads them if its
  // weights turn out to need them.
  __device__ __forceinline__ void load_row(long row0, int t0, ChunkData<KB, VB, GP> &c, bool vskip = false) const {
    const int rows = row0 < 0 ? 0 : min(capacity - t0, kChunk);
    row0 = row0 < 0 ? 0L : row0;
    const auto rk = rsrc(kbase + row0 * kRowBytes, rows * kRowBytes);
    const auto rkn = rsrc(knbase + row0 * 4, rows * 4);
    const auto rv = rsrc(vbase + row0 * kVRow, vskip ? 0 : rows * kVRow);
    const auto rvn = rsrc(vnbase + row0 * 4, rows * 4);
    c.vskip = vskip;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mo = m * 16 * kRowBytes;
      if (KB == 3) {
        typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
        const u32x3_t w = __builtin_amdgcn_raw_buffer_load_b96(rk, koff + mo, 0, 0);
        c.k[m][0] = w[0]; c.k[m][1] = w[1]; c.k[m][2] = w[2];
      } else if (KB == 2) {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(rk, koff + mo, 0, 0);
        c.k[m][0] = w[0]; c.k[m][1] = w[1];
      } else {
#pragma unroll
        for (int i = 0; i < ChunkData<KB, VB, GP>::kw; i += 4) {
          const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + mo + 4 * i, 0, 0);
          c.k[m][i] = w[0]; c.k[m][i + 1] = w[1]; c.k[m][i + 2] = w[2]; c.k[m][i + 3] = w[3];
        }
      }
    }
    if (NV == 2) {
      if (KB) {
        const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(rkn, knoff, 0, 0);
        c.kn[0] = __uint_as_float(a[0]); c.kn[1] = __uint_as_float(a[1]);
      }
      const u32x2_t b = __builtin_amdgcn_raw_buffer_load_b64(rvn, knoff, 0, 0);
      c.vn[0] = __uint_as_float(b[0]); c.vn[1] = __uint_as_float(b[1]);
    } else {
      if (KB) {
        const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(rkn, knoff, 0, 0);
#pragma unroll
        for (int j = 0; j < NV; ++j) c.kn[j] = __uint_as_float(a[j]);
      }
      const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(rvn, knoff, 0, 0);
#pragma unroll
      for (int j = 0; j < NV; ++j) c.vn[j] = __uint_as_float(b[j]);
    }
    load_v(rv, c.v);
  }

  // The V data of the lane's 8 position slots: one code word, (2-bit) the
  // dword holding the 16 bits of coordinates 8 col .. 8 col + 7, (3-bit) the
  // two dwords holding their 24 bits, or (INT8) their 8 bytes.
  __device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t rv, uint32_t (&v)[ChunkData<KB, VB, GP>::kvw]) const {
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const uint32_t off = voff + (16 * (s8 >> 2) + (s8 & 3)) * kVRow;
      if (VB == 3 || VB == kInt8) {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0);
        v[2 * s8] = w[0];
        v[2 * s8 + 1] = w[1];
      } else {
        v[s8] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0);
      }
    }
  }

  // Scores of the chunk in D layout (lane: slots 4 m + r, head col).
  __device__ __forceinline__ void score(const ChunkData<KB, VB, GP> &c, float (&s)[8]) const {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (KB == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const half8_t a = as_half8(c.k[m][4 * q], c.k[m][4 * q + 1], c.k[m][4 * q + 2], c.k[m][4 * q + 3]);
          acc = mma(a, bq[q], acc);
        }
      } else if (KB == kInt8) {
        // the lane's 32 bytes are coordinates 32 grp .. 32 grp + 31; step q
        // takes 8 of them, widened exactly to fp16 (one MFMA: exact A)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w0 = c.k[m][2 * q] ^ 0x80808080u, w1 = c.k[m][2 * q + 1] ^ 0x80808080u;
          const half8_t a = as_half8(i8_pair_exact<0>(w0), i8_pair_exact<2>(w0), i8_pair_exact<0>(w1),
                                     i8_pair_exact<2>(w1));
          acc = mma(a, bq[q], acc);
        }
      } else if (KB == 2) {
        // the lane's 32 coordinates are 64 bits; step q takes coordinates
        // 8 q .. 8 q + 7, the four nibbles (code pairs) 4 (q & 1) .. + 3 of
        // word q / 2, each the low nibble of a byte of the word or of the
        // word shifted right by 4
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = c.k[m][q >> 1], ws = w >> 4;
          uint32_t ad[4];
          if (q & 1) {
            ad[0] = baddr<2>(w, rep4); ad[1] = baddr<2>(ws, rep4);
            ad[2] = baddr<3>(w, rep4); ad[3] = baddr<3>(ws, rep4);
          } else {
            ad[0] = baddr<0>(w, rep4); ad[1] = baddr<0>(ws, rep4);
            ad[2] = baddr<1>(w, rep4); ad[3] = baddr<1>(ws, rep4);
          }
          const half8_t ah = as_half8(lds_at<0>(lds, ad[0]), lds_at<0>(lds, ad[1]), lds_at<0>(lds, ad[2]),
                                      lds_at<0>(lds, ad[3]));
          const half8_t al = as_half8(lds_at_sep<kKloOff>(lds, ad[0]), lds_at_sep<kKloOff>(lds, ad[1]),
                                      lds_at_sep<kKloOff>(lds, ad[2]), lds_at_sep<kKloOff>(lds, ad[3]));
          acc = mma(ah, bq[q], acc);
          acc = mma(al, bq[q], acc);
        }
      } else if (KB == 3) {
        // byte addresses of the 16 code pairs of the lane's 32 coordinates:
        // pair j sits at bit 6 j of the 96-bit stream w2:w1:w0, which is
        // byte 0 or 3 of one of the windows below (stream shifted right by
        // 0, 6, 12, 18, 48, 54, 60, 66 bits)
        uint32_t ad[16];
        const uint32_t w0 = c.k[m][0], w1 = c.k[m][1], w2 = c.k[m][2];
        const uint32_t x6 = __builtin_amdgcn_alignbit(w1, w0, 6), x12 = __builtin_amdgcn_alignbit(w1, w0, 12);
        const uint32_t x18 = __builtin_amdgcn_alignbit(w1, w0, 18), x48 = __builtin_amdgcn_alignbit(w2, w1, 16);
        const uint32_t x54 = __builtin_amdgcn_alignbit(w2, w1, 22), x60 = __builtin_amdgcn_alignbit(w2, w1, 28);
        const uint32_t x66 = w2 >> 2;
        ad[0] = baddr<0>(w0, rep4);
        ad[1] = baddr<0>(x6, rep4);
        ad[2] = baddr<0>(x12, rep4);
        ad[3] = baddr<0>(x18, rep4);
        ad[4] = baddr<3>(w0, rep4);
        ad[5] = baddr<3>(x6, rep4);
        ad[6] = baddr<3>(x12, rep4);
        ad[7] = baddr<3>(x18, rep4);
        ad[8] = baddr<0>(x48, rep4);
        ad[9] = baddr<0>(x54, rep4);
        ad[10] = baddr<0>(x60, rep4);
        ad[11] = baddr<0>(x66, rep4);
        ad[12] = baddr<3>(x48, rep4);
        ad[13] = baddr<3>(x54, rep4);
        ad[14] = baddr<3>(x60, rep4);
        ad[15] = baddr<3>(x66, rep4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const half8_t ah = as_half8(lds_at<0>(lds, ad[4 * q]), lds_at<0>(lds, ad[4 * q + 1]),
                                      lds_at<0>(lds, ad[4 * q + 2]), lds_at<0>(lds, ad[4 * q + 3]));
          const half8_t al = as_half8(lds_at_sep<kKloOff>(lds, ad[4 * q]), lds_at_sep<kKloOff>(lds, ad[4 * q + 1]),
                                      lds_at_sep<kKloOff>(lds, ad[4 * q + 2]), lds_at_sep<kKloOff>(lds, ad[4 * q + 3]));
          acc = mma(ah, bq[q], acc);
          acc = mma(al, bq[q], acc);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = c.k[m][q];
          const uint32_t a0 = baddr<0>(w, rep4), a1 = baddr<1>(w, rep4);
          const uint32_t a2 = baddr<2>(w, rep4), a3 = baddr<3>(w, rep4);
          const half8_t ah = as_half8(lds_at<0>(lds, a0), lds_at<0>(lds, a1), lds_at<0>(lds, a2), lds_at<0>(lds, a3));
          const half8_t al = as_half8(lds_at_sep<kKloOff>(lds, a0), lds_at_sep<kKloOff>(lds, a1),
                                      lds_at_sep<kKloOff>(lds, a2), lds_at_sep<kKloOff>(lds, a3));
          acc = mma(ah, bq[q], acc);
          acc = mma(al, bq[q], acc);
        }
      }
      // column h + GP holds the lo half of head h's query: fold it in
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * m + r] = acc[r] + dpp_f<kRowShl + GP, 0xf>(0.0f, acc[r]);
    }
  }

  // D layout -> compact layout (see the struct comment).
  __device__ __forceinline__ void compact(const float (&s)[8], float (&c)[NV]) const {
    if (GP == 4) {
      c[0] = s[0];
      c[1] = s[1];
      c[0] = dpp_f<kRowShr + 4, 0x2>(c[0], s[2]);
      c[1] = dpp_f<kRowShr + 4, 0x2>(c[1], s[3]);
      c[0] = dpp_f<kRowShr + 8, 0x4>(c[0], s[4]);
      c[1] = dpp_f<kRowShr + 8, 0x4>(c[1], s[5]);
      c[0] = dpp_f<kRowShr + 12, 0x8>(c[0], s[6]);
      c[1] = dpp_f<kRowShr + 12, 0x8>(c[1], s[7]);
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) c[j] = s[j];
      c[0] = dpp_f<kRowShr + 8, 0xc>(c[0], s[4]);
      c[1] = dpp_f<kRowShr + 8, 0xc>(c[1], s[5]);
      c[2] = dpp_f<kRowShr + 8, 0xc>(c[2], s[6]);
      c[3] = dpp_f<kRowShr + 8, 0xc>(c[3], s[7]);
    }
  }

  // Compact hi/lo weight pairs -> A operand of the value MFMA.  Row r of A
  // (lane column r) is P_hi of head r for r < GP, P_lo of head r - GP for
  // GP <= r < 2 GP, zero beyond; word s2 holds slots 2 s2, 2 s2 + 1, which
  // compact lane (grp, GP kc + h) holds for kc = 2 s2 / NV.
  __device__ __forceinline__ half8_t weights_operand(const uint32_t (&wh)[NV / 2], const uint32_t (&wl)[NV / 2]) const {
    uint32_t x[4];
    if (GP == 4) {
      // hi rows (banks 0): source lane + 4 s2; lo rows (bank 1): source lane + 4 s2 - 4
      x[0] = dpp_bank<kRowShl + 0, 0x1>(0u, wh[0]);
      x[0] = dpp_bank<kRowShr + 4, 0x2>(x[0], wl[0]);
      x[1] = dpp_bank<kRowShl + 4, 0x1>(0u, wh[0]);
      x[1] = dpp_bank<kRowShl + 0, 0x2>(x[1], wl[0]);
      x[2] = dpp_bank<kRowShl + 8, 0x1>(0u, wh[0]);
      x[2] = dpp_bank<kRowShl + 4, 0x2>(x[2], wl[0]);
      x[3] = dpp_bank<kRowShl + 12, 0x1>(0u, wh[0]);
      x[3] = dpp_bank<kRowShl + 8, 0x2>(x[3], wl[0]);
    } else {
      // hi rows (banks 0, 1): source lane + 8 kc; lo rows (banks 2, 3): source lane + 8 kc - 8
      x[0] = dpp_bank<kRowShl + 0, 0x3>(0u, wh[0]);
      x[0] = dpp_bank<kRowShr + 8, 0xc>(x[0], wl[0]);
      x[1] = dpp_bank<kRowShl + 0, 0x3>(0u, wh[1]);
      x[1] = dpp_bank<kRowShr + 8, 0xc>(x[1], wl[1]);
      x[2] = dpp_bank<kRowShl + 8, 0x3>(0u, wh[0]);
      x[2] = dpp_bank<kRowShl + 0, 0xc>(x[2], wl[0]);
      x[3] = dpp_bank<kRowShl + 8, 0x3>(0u, wh[1]);
      x[3] = dpp_bank<kRowShl + 0, 0xc>(x[3], wl[1]);
    }
    return as_half8(x[0], x[1], x[2], x[3]);
  }

  // Scale the value accumulators of each head by its own factor (compact
  // lane h holds head h's factor): rows r of lane group g belong to head r
  // (GP = 4) or 4 (g & 1) + r (GP = 8).
  __device__ __forceinline__ void scale_heads(float f) {
    float fr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), r));
      if (GP == 4) {
        fr[r] = lo;
      } else {
        const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 4 + r));
        fr[r] = (grp & 1) ? hi : lo;
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) accv[q][r] *= fr[r];
    }
  }

  // Online softmax on compact scores (base-2 logits; -inf = masked).  The
  // accumulators are only rescaled when the running maximum grows by more
  // than 2^8.  Returns the value MFMA's A operand: P = p n vscale as hi and lo
  // fp16 rows (n: the positions' V norms, 1 for fp16 rows).
  //
  // The value scale (SCALED): P must fit fp16 (below 2^16) and the largest
  // terms of a head must stay far above fp16's subnormal range (2^-14),
  // whatever the spread of the norms.  vscale is a power of two per head, so
  // dividing it out at the end is exact.  It is lowered when a
  // weight-times-norm of the chunk would give P > 2^15 (to 16 / the head's
  // largest p n, rounded up to a power of two, so that term lands in
  // (8, 16]), and raised by 2^floor(growth) when the head's running maximum
  // grows (its earlier terms shrink by 2^-growth), up to 2^40.  The 2^11
  // headroom above 16 exceeds the 2^8 by which a weight may outgrow the lazily
  // updated maximum, so lowering is rare.  The largest term of a head
  // therefore stays within [2^2, 2^15], where hi and lo carry full
  // precision, unless the head's largest weights fall on rows of zero norm
  // and every other weight is below 2^-30 of them; a row whose V norm is
  // tiny next to others does not force the scale down unless its weight is
  // large too.
  // HMAX: every chunk's maximum per head is needed (sparse-V); otherwise
  // the head's maximum is only formed when some lane's values outgrow the
  // running maximum by the rescale margin (the same decisions: a head's
  // maximum grows past it exactly when one of its lanes' does).
  template <bool TAIL, bool SCALED, bool HMAX>
  __device__ __forceinline__ half8_t softmax(const float (&c)[NV], const float (&n)[NV]) {
    // c holds the logits before the query's power-of-two scale qinv (> 0),
    // which commutes with the maximum and enters the exponent by an fma
    float cmax = c[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) cmax = fmaxf(cmax, c[j]);
    cmax *= qinv;  // exact (a power of two), so it commutes with the maximum
    if (HMAX) cmax = head_max<GP>(cmax);
    bool grow = cmax > m_run + kRescale;
    if (!HMAX && __ballot(grow)) {
      cmax = head_max<GP>(cmax);
      grow = cmax > m_run + kRescale;
    }
    chunk_max = cmax;
    if (__ballot(grow)) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      float f = alpha;
      if (SCALED && grow) {
        // raise the scale by the power of two the maximum grew by (a first
        // maximum, m_run = -inf, leaves it at its initial 2^40)
        const float up = fminf(ldexpf(1.0f, static_cast<int>(fminf(m_new - m_run, 64.0f))), kVscaleMax / vscale);
        vscale *= up;
        f *= up;
      }
      m_run = m_new;
      l_run *= alpha;
      scale_heads(f);
    }
    float p[NV], P[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      p[j] = __builtin_amdgcn_exp2f(fmaf(c[j], qinv, -m_run));
      if (TAIL) p[j] = (c[j] == -INFINITY) ? 0.0f : p[j];
      l_run += p[j];
      P[j] = p[j] * n[j];
    }
    if (SCALED) {
      float lm = P[0];
#pragma unroll
      for (int j = 1; j < NV; ++j) lm = fmaxf(lm, P[j]);
      if (__ballot(lm * vscale > 32768.0f)) {
        // lower the scale of the heads whose largest p n asks for it (the
        // whole wave runs this, as scale_heads reads other lanes)
        const float hm = head_max<GP>(lm);
        const float vs = (hm * vscale > 32768.0f) ? 16.0f / pow2_ceil(hm) : vscale;
        const float f = vs / vscale;
        vscale = vs;
        scale_heads(f);
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) P[j] *= vscale;
    }
    uint32_t wh[NV / 2], wl[NV / 2];
#pragma unroll
    for (int j = 0; j < NV; j += 2) split_pair(P[j], P[j + 1], wh[j / 2], wl[j / 2]);
    return weights_operand(wh, wl);
  }

  // Optional raw scores (natural-log units) of the real heads.
  template <bool TAIL>
  __device__ __forceinline__ void store_scores(int t0, int we, const float (&c)[NV], float *scores,
                                               long score_row0, int length) const {
    const int h = col % GP;
    if (h < G) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int t = t0 + cpos + j;
        if (!TAIL || t < we) scores[(score_row0 + h) * length + t] = c[j] * qinv * kLn2;
      }
    }
  }

  // Packed values: pair the nibbles of slots 2 s2 and 2 s2 + 1 per byte (one
  // byte per coordinate pair index), then per tile q one table lookup per
  // slot pair and one MFMA: D[(head, hi/lo)][coordinate 8 col + q] +=
  // P[(head, hi/lo)][slot] * c[code of slot, coordinate].
  __device__ __forceinline__ void values(const uint32_t (&cv)[ChunkData<KB, VB, GP>::kvw], const half8_t ap) {
    if (KB == kInt8) {
      // INT8: slot s holds bytes 8 col .. 8 col + 7 in words 2 s, 2 s + 1;
      // tile q takes byte q % 4 of word q / 4 of every slot, two slots an
      // operand word, as x 2^-10 (the merge multiplies by 2^10)
      uint32_t x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = cv[i] ^ 0x80808080u;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t a4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t a = x[4 * u + (q >> 2)], b = x[4 * u + 2 + (q >> 2)];
          switch (q & 3) {
            case 0: a4[u] = i8_cross_pair<0>(a, b); break;
            case 1: a4[u] = i8_cross_pair<1>(a, b); break;
            case 2: a4[u] = i8_cross_pair<2>(a, b); break;
            default: a4[u] = i8_cross_pair<3>(a, b); break;
          }
        }
        accv[q] = mma(ap, as_half8(a4[0], a4[1], a4[2], a4[3]), accv[q]);
      }
      return;
    }
    if (VB == 2) {
      // 2-bit codes: per slot pair, the 4-bit pairs (slot 2 s2 low) of the
      // even coordinates of both 16-bit halves of the words (ev) and of the
      // odd ones (od); the lane's half of each goes into one word (even
      // coordinates in bytes 0, 1, odd in bytes 2, 3), where coordinate
      // 8 col + q is nibble q / 2 (q even) or 4 + q / 2 (q odd): the low
      // nibble of a byte of the word, or of the word shifted right by 4
      uint32_t pw[4], ps[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const uint32_t x0 = cv[2 * s2], x1 = cv[2 * s2 + 1];
        const uint32_t ev = bfi(0x33333333u, x0, x1 << 2), od = bfi(0x33333333u, x0 >> 2, x1);
        pw[s2] = __builtin_amdgcn_perm(od, ev, vsh);
        ps[s2] = pw[s2] >> 4;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // nibble n = q / 2 + 4 (q & 1): byte n / 2 of pw (n even) or ps (n odd)
        const int n = (q >> 1) + 4 * (q & 1);
        const uint32_t *src = (n & 1) ? ps : pw;
        uint32_t a4[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const uint32_t w = src[s2];
          uint32_t ad;
          switch (n >> 1) {
            case 0: ad = two_tables<KB, VB>() ? baddr_hi<0>(w, rep4v) : baddr<0>(w, rep4); break;
            case 1: ad = two_tables<KB, VB>() ? baddr_hi<1>(w, rep4v) : baddr<1>(w, rep4); break;
            case 2: ad = two_tables<KB, VB>() ? baddr_hi<2>(w, rep4v) : baddr<2>(w, rep4); break;
            default: ad = two_tables<KB, VB>() ? baddr_hi<3>(w, rep4v) : baddr<3>(w, rep4); break;
          }
          a4[s2] = lds_at<0>(lds, ad);
        }
        accv[q] = mma(ap, as_half8(a4[0], a4[1], a4[2], a4[3]), accv[q]);
      }
      return;
    }
    if (VB == 3) {
      // 3-bit codes: the lane's 24 bits of each slot (coordinate 8 col + k
      // at bit 3 k), then per slot pair the 6-bit pairs (slot 2 s2 low,
      // slot 2 s2 + 1 high) of the even coordinates at bits 0, 6, 12, 18
      // (ev) and of the odd ones (od); pair j is byte 0 of the word shifted
      // right by 6 j, and the table ignores the byte's top 2 bits
      uint32_t ev[4], od[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const uint32_t fa = __builtin_amdgcn_alignbit(cv[4 * s2 + 1], vlast ? cv[4 * s2 + 1] : cv[4 * s2], vsh);
        const uint32_t fb = __builtin_amdgcn_alignbit(cv[4 * s2 + 3], vlast ? cv[4 * s2 + 3] : cv[4 * s2 + 2], vsh);
        ev[s2] = bfi(0x1c71c7u, fa, fb << 3);
        od[s2] = bfi(0x1c71c7u, fa >> 3, fb);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t *src = (q & 1) ? od : ev;
        uint32_t a4[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const uint32_t w = src[s2] >> (6 * (q >> 1));
          a4[s2] = lds_at<0>(lds, two_tables<KB, VB>() ? baddr_hi<0>(w, rep4v) : baddr<0>(w, rep4));
        }
        accv[q] = mma(ap, as_half8(a4[0], a4[1], a4[2], a4[3]), accv[q]);
      }
      return;
    }
    uint32_t ev[4], od[4];  // bytes j: coordinates 8 col + 2 j (ev) and 8 col + 2 j + 1 (od)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const uint32_t x0 = cv[2 * s2], x1 = cv[2 * s2 + 1];
      ev[s2] = bfi(0x0f0f0f0fu, x0, x1 << 4);
      od[s2] = bfi(0x0f0f0f0fu, x0 >> 4, x1);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t *src = (q & 1) ? od : ev;
      uint32_t a4[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const uint32_t w = src[s2];
        uint32_t ad;
        if (two_tables<KB, VB>()) {
          switch (q >> 1) {
            case 0: ad = baddr_hi<0>(w, rep4v); break;
            case 1: ad = baddr_hi<1>(w, rep4v); break;
            case 2: ad = baddr_hi<2>(w, rep4v); break;
            default: ad = baddr_hi<3>(w, rep4v); break;
          }
        } else {
          switch (q >> 1) {
            case 0: ad = baddr<0>(w, rep4); break;
            case 1: ad = baddr<1>(w, rep4); break;
            case 2: ad = baddr<2>(w, rep4); break;
            default: ad = baddr<3>(w, rep4); break;
          }
        }
        a4[s2] = lds_at<0>(lds, ad);
      }
      accv[q] = mma(ap, as_half8(a4[0], a4[1], a4[2], a4[3]), accv[q]);
    }
  }

  // One chunk of packed positions [t0, t0 + 32); positions >= we are masked.
  template <bool TAIL, bool SP>
  __device__ __forceinline__ void cold_chunk(int t0, int we, const ChunkData<KB, VB, GP> &c, float *scores,
                                             long score_row0, int length) {
    float s[8], cs[NV];
    score(c, s);
    compact(s, cs);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (KB) cs[j] *= c.kn[j];
      if (TAIL && t0 + cpos + j >= we) cs[j] = -INFINITY;
    }
    if (scores) store_scores<TAIL>(t0, we, cs, scores, score_row0, length);
    const half8_t ap = softmax<TAIL, true, SP>(cs, c.vn);
    if (!SP) {
      // exact decode: a threshold never set (kept as a runtime test: the
      // branch keeps the value phase out of the score phase's schedule)
      if (sparse_lg != -INFINITY && !__ballot(chunk_max - m_run >= sparse_lg)) return;
    } else {
      // sparse-V: every weight of the chunk, for every real head, below the
      // threshold times the larger of the wave's running maximum and the
      // block maximum after the first round of chunks (neither exceeds the
      // final maximum, and both are the same on every call): the chunk's
      // values are skipped; its weights stay in the sum
      const float r = fmaxf(m_run, block_ref);
      const bool skip = !__ballot(col % GP < G && chunk_max - r >= sparse_lg);
      pred_skip = skip;
      if (skip) return;
      if (c.vskip) {
        // predicted skippable, but needed: load the V codes now
        const long row0 = row_of(t0);
        const int rows = row0 < 0 ? 0 : min(capacity - t0, kChunk);
        const auto rv = rsrc(vbase + (row0 < 0 ? 0L : row0) * kVRow, rows * kVRow);
        uint32_t vv[ChunkData<KB, VB, GP>::kvw];
        load_v(rv, vv);
        values(vv, ap);
        return;
      }
    }
    values(c.v, ap);
  }

  // sparse-V: the waves' running maxima after their first chunk, exchanged
  // at a block barrier (every wave has a first chunk when this is called)
  __device__ __forceinline__ void exchange_max() {
    typedef __attribute__((address_space(3))) const volatile u32x4_t lds_v4;
    typedef __attribute__((address_space(3))) volatile float lds_f;
    const uint32_t base = bmax_at;
    if (col < GP && grp == 0) *reinterpret_cast<lds_f *>(base + 4u * (16u * col + wave_id)) = m_run;
    __syncthreads();
    float r = block_ref;
#pragma unroll
    for (int i = 0; i < kMaxWaves / 4; ++i) {
      // head h's maxima are floats 16 h .. 16 h + 15 (one per wave)
      const u32x4_t m = *reinterpret_cast<lds_v4 *>(base + 64u * (col % GP) + 16u * i);
      r = fmaxf(r, fmaxf(fmaxf(__uint_as_float(m[0]), __uint_as_float(m[1])),
                         fmaxf(__uint_as_float(m[2]), __uint_as_float(m[3]))));
    }
    block_ref = r;
  }

  // One chunk of the fp16 hot window (delegated V), positions >= we masked.
  // Chunk [t0, t0 + 32) of the fp16 hot window [wb, we): t0 is on the
  // 32-position grid (a paged chunk then lies in one block), and positions
  // outside the window are masked.
  __device__ __forceinline__ void hot_chunk(int t0, int wb, int we, const ChunkData<KB, VB, GP> &c, float *scores,
                                            long score_row0, int length) {
    float s[8], cs[NV], vn[NV];
    score(c, s);
    compact(s, cs);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (KB) cs[j] *= c.kn[j];
      vn[j] = 1.0f;
      const int t = t0 + cpos + j;
      if (t < wb || t >= we) cs[j] = -INFINITY;
    }
    if (scores && col % GP < G) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int t = t0 + cpos + j;
        if (t >= wb && t < we) scores[(score_row0 + col % GP) * length + t] = cs[j] * qinv * kLn2;
      }
    }
    const half8_t ap = softmax<true, false, false>(cs, vn);
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
      accv[q] = mma(ap, as_half8(u[0], u[1], u[2], u[3]), accv[q]);
    }
  }

  // Write this wave's partial result of the real heads (h < G) into its
  // merge slot [GP][kPS]: (max, sum, 1 / vscale, 0), then the accumulator in
  // coordinate order (`hot_layout` selects the value tiles' coordinate map).
  // The hi and lo rows of the value accumulators sit in partner lane groups
  // (GP = 4: groups 0 / 1 hold rows 0-3 / 4-7, i.e. hi / lo of heads 0-3;
  // GP = 8: groups 0, 1 / 2, 3 hold hi / lo of heads 0-3, 4-7).  One lane
  // swap of rows r and r + 2 brings each lane the hi and lo of one head:
  // after swapping and adding, lane group g holds heads h0 + e (e = 0 from
  // rows 0 and 2, e = 1 from rows 1 and 3), which the lane then writes.
  __device__ __forceinline__ void to_slot(float *slot_base, bool hot_layout) const {
    // the lane index is recomputed here: reusing the prologue's lane
    // offsets would keep them live (in registers) across the main loop
    uint32_t lid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
    const int col = lid & 15, grp = lid >> 4;
    const float l_wave = head_sum<GP>(l_run);
    if (col < G && grp == 0) {
      // 1 / vscale, exactly (vscale is a power of two)
      int ex;
      (void)frexpf(vscale, &ex);
      *reinterpret_cast<float4 *>(slot_base + col * kPS) = make_float4(m_run, l_wave, ldexpf(1.0f, 1 - ex), 0.0f);
    }
    const int h0 = (GP == 4) ? 2 * (grp & 1) : 4 * (grp & 1) + 2 * (grp >> 1);
    float v[2][8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t x = __float_as_uint(accv[q][e]), y = __float_as_uint(accv[q][e + 2]);
        const u32x2_t sw = (GP == 4) ? __builtin_amdgcn_permlane16_swap(x, y, false, false)
                                     : __builtin_amdgcn_permlane32_swap(x, y, false, false);
        v[e][q] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
    }
    if (GP == 4 && grp >= 2) return;  // padding rows
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int h = h0 + e;
      if (h < G) {
        float *dst = slot_base + h * kPS + kPV;
        if (hot_layout) {
#pragma unroll
          for (int q = 0; q < 8; ++q) dst[16 * q + col] = v[e][q];
        } else {
          *reinterpret_cast<float4 *>(dst + 8 * col) = make_float4(v[e][0], v[e][1], v[e][2], v[e][3]);
          *reinterpret_cast<float4 *>(dst + 8 * col + 4) = make_float4(v[e][4], v[e][5], v[e][6], v[e][7]);
        }
      }
    }
  }
};

// Merge the NW wave slots [w][GP][kPS] of head h, values 4 j4 .. 4 j4 + 3:
// hdr = (max M, sum, 0, 0), val = sum_w 2^(m_w - M) acc_w / vscale_w.  A
// wave that saw no position of the head has m_w = -inf and weighs 0.
template <int NW, int GP>
__device__ __forceinline__ void merge_slots(const float *slots, int h, int j4, float4 &hdr, float4 &val) {
  float4 st[NW];
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    st[w] = *reinterpret_cast<const float4 *>(slots + (w * GP + h) * kPS);
    M = fmaxf(M, st[w].x);
  }
  float L = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float4 a = *reinterpret_cast<const float4 *>(slots + (w * GP + h) * kPS + kPV + 4 * j4);
    const float e = (st[w].x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st[w].x - M);
    L += e * st[w].y;
    const float f = e * st[w].z;
    acc.x += f * a.x;
    acc.y += f * a.y;
    acc.z += f * a.z;
    acc.w += f * a.w;
  }
  hdr = make_float4(M, L, 0.0f, 0.0f);
  val = acc;
}

__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  const u32x4_t u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, kCoherentLoad);
}

// Issue priority 0..3 from a wave-uniform value (clamped).
__device__ __forceinline__ void set_priority(int k) {
  if (k >= 3) {
    __builtin_amdgcn_s_setprio(3);
  } else if (k == 2) {
    __builtin_amdgcn_s_setprio(2);
  } else if (k == 1) {
    __builtin_amdgcn_s_setprio(1);
  } else {
    __builtin_amdgcn_s_setprio(0);
  }
}

// Wave balancing.  The instruction arbiter of a SIMD favours the oldest of
// its waves, so with equal shares of chunks the oldest wave finishes far
// ahead and the youngest runs alone at the end, without other waves to hide
// its latencies.  Each wave therefore publishes how many chunks (fp16 K) or
// pairs of chunks (packed and INT8 K) it has done and runs at a priority
// equal to how far it lags the leading wave of the block.  Only the issue
// order changes: which wave takes which chunk, and so every sum, stays the
// same.
// The counters live at LDS byte address PROG (the kernel's only LDS array
// starts at address 0); volatile LDS-space accesses, so every step reads
// the other waves' current counts with ds_read.
template <int NW, uint32_t PROG>
struct Balance {
  typedef __attribute__((address_space(3))) volatile int lds_int;
  typedef __attribute__((address_space(3))) const volatile u32x4_t lds_u32x4;
  int done = 0;
  // this wave finished a chunk: publish its count, then set its priority
  // from the counts of all waves
  __device__ __forceinline__ void step(int wave, int lane) {
    ++done;
    if (lane == 0) *reinterpret_cast<lds_int *>(PROG + 4u * wave) = done;
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < NW; w += 4) {
      const u32x4_t c = *reinterpret_cast<lds_u32x4 *>(PROG + 4u * w);
      m = max(m, max(max(c[0], c[1]), max(c[2], c[3])));
    }
    set_priority(static_cast<int>(__builtin_amdgcn_readfirstlane(m)) - done);
  }
};

// AP: the fused append (tq_decode_attention_append; exact decode, no scores).
template <int KB, int VB, int GP, bool PG, bool SC, bool SP, bool AP>
__global__ __launch_bounds__(64 * waves_of<KB>(), 1) void decode_mfma_kernel(const DecodeParams p) {
  constexpr int kWaves = waves_of<KB>();
  constexpr int kThreads = 64 * kWaves;
  using L = Lay<KB, VB, GP>;
  using WaveT = Wave<KB, VB, GP, PG>;
  constexpr int NV = WaveT::NV;
  // Static LDS: its base address is a compile-time constant, so table reads
  // fold the table offset into the instruction.
  __shared__ __align__(16) uint32_t lds[L::total];
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (the wave's range of
  // positions, the buffer descriptors) then stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // A query group of more than 8 heads runs as head groups of 8 (the last
  // one possibly smaller): each is a unit of its own (its splits, partials
  // and arrival counter) that reads its KV head's rows.  G is this block's
  // head count, Gs the partial stride (8, or the whole group when smaller).
  const int g_all = p.q_heads / p.kv_heads;
  const int n_hg = (g_all + 7) / 8;
  const int Gs = min(g_all, 8);
  // SC: the launch writes the scaled logits (parity runs); otherwise their
  // address arithmetic is compiled out
  float *const scores = SC ? p.scores : nullptr;
  float *qw = reinterpret_cast<float *>(lds + L::qwork);
  int *flag = reinterpret_cast<int *>(lds + L::red);
  int *prog = reinterpret_cast<int *>(lds + L::prog);
  float *work = reinterpret_cast<float *>(lds);  // merge area after the main loop
  float *slots = reinterpret_cast<float *>(lds + L::slots);

  const int nsplit = p.n_cold_splits;
  const int vunit = blockIdx.x / nsplit;  // (KV unit, head group)
  const int split = blockIdx.x % nsplit;
  const int unit = vunit / n_hg;          // (batch, KV head)
  const int hgrp = vunit % n_hg;
  const int G = min(g_all - 8 * hgrp, 8);
  const int b = unit / p.kv_heads;
  const int kv = unit % p.kv_heads;
  const long hq0 = static_cast<long>(b) * p.q_heads + static_cast<long>(kv) * g_all + 8 * hgrp;
  const int s0 = split * p.cold_split_len;
  const int s1 = min(p.cold_len, s0 + p.cold_split_len);
  const int span = max(0, s1 - s0);
  // chunks of 32 positions of the split, dealt round-robin to the waves
  // (wave w takes chunks w, w + kWaves, ...): balanced to one chunk, and
  // the same assignment, hence the same sums, on every call
  const int n_chunks = (span + kChunk - 1) / kChunk;
  const int n_full = span / kChunk;

  constexpr bool k_rot = rotated_k<KB>();
  constexpr int kRowBytes = WaveT::kRowBytes;
  constexpr int kVRow = WaveT::kVRow;
  WaveT W;
  W.col = lane & 15;
  W.grp = lane >> 4;
  {
    const int i0 = NV * (W.col / GP);  // first compact slot
    W.cpos = 16 * (i0 >> 2) + 4 * W.grp + (i0 & 3);
  }
  W.rep4 = (lane & 31) * 4u;
  W.rep4v = W.rep4 + v_table_byte<KB, VB>();
  W.lds = lds;
  W.G = G;
  // contiguous: the unit's rows start at unit * capacity; paged: load()
  // finds each chunk's block
  const long rowbase = PG ? 0L : static_cast<long>(unit) * p.capacity;
  W.pg = p.pg;
  W.unit = unit;
  W.kbase = KB ? reinterpret_cast<const char *>(p.k.codes) + rowbase * kRowBytes
               : reinterpret_cast<const char *>(p.k.fp16) + rowbase * kRowBytes;
  W.knbase = KB ? reinterpret_cast<const char *>(p.k.norms + rowbase) : W.kbase;
  W.vbase = reinterpret_cast<const char *>(p.v.codes) + rowbase * kVRow;
  W.vnbase = reinterpret_cast<const char *>(p.v.norms + rowbase);
  W.koff = static_cast<uint32_t>(W.col * kRowBytes + W.grp * (kRowBytes / 4));
  W.knoff = static_cast<uint32_t>(4 * W.cpos);
  // 3-bit V: the lane's 24 bits start at byte 3 col of the row, in dword
  // 3 col / 4 at bit 8 (3 col % 4); lane 15 reads dwords 10 and 11 (the
  // row's last two) and takes its bits from the second
  // 2-bit V: its 16 bits are half h = col % 2 of dword col / 2, picked
  // after the pairing by a v_perm selector (bytes 2 h, 2 h + 1 of each word)
  W.voff = static_cast<uint32_t>(W.grp * 4 * kVRow +
                                 (VB == 3 ? 4 * min(3 * W.col / 4, 10) : VB == 2 ? 4 * (W.col / 2) : W.col * (kVRow / 16)));
  W.vsh = VB == 2 ? ((W.col & 1) ? 0x07060302u : 0x05040100u) : 8u * ((3u * W.col) & 3u);
  W.vlast = W.col == 15;
  W.capacity = p.capacity;
  W.hot_len = p.v.hot > 0 ? p.v.hot : 1;
  W.ring = (p.v.mode == TQ_SIDE_DELEGATED) ? p.v.fp16 + static_cast<long>(unit) * p.v.hot * D : nullptr;
  W.vscale = kVscaleMax;
  W.sparse_lg = p.sparse_lg;
  W.pred_skip = false;
  W.bmax_at = 4u * L::bmax;
  W.wave_id = wave;
  W.block_ref = -INFINITY;
  W.reset();

  // ---- the query, then the first chunk, in flight while the block builds
  // its tables.  Wave h < G takes query head h, coordinates lane and
  // lane + 64.  The query is issued first: waiting for it (loads complete
  // in issue order) then does not wait for the chunk.
  // (Both loads are unconditional, so the wait for the query can count
  // the chunk's loads as still outstanding: waves past G read head G - 1,
  // waves past the split read an empty range, which returns zeros.)
  uint32_t qa_raw = p.q[(hq0 + min(wave, G - 1)) * D + lane];  // fp16 bits
  uint32_t qb_raw = p.q[(hq0 + min(wave, G - 1)) * D + lane + 64];
  // fused append: in the split holding the new position, the wave that
  // reads the position's chunk (chunk c goes to wave c % kWaves) writes the
  // new K and V rows first and waits for the stores, so it reads them back;
  // no other wave reads that chunk, so nothing else waits.  Every head group
  // of the unit writes the same rows.
  // When the position lies in a later chunk of that wave, the wave's first
  // chunk load goes out first and the append runs while it is in flight.
  // The new rows' loads go out before the wave's first chunk load (so the
  // append does not wait for the chunk).  When the position lies in a later
  // chunk of the wave, the rows are written after the prologue (whose block
  // barrier the append would otherwise hold up), before the main loop.
  static_assert(!(AP && (SP || SC)), "the fused append runs the exact decode without scores");
  const int ap_chunk = (AP && split == p.ap_split) ? (p.ap_offset - s0) / kChunk : -1;
  const bool ap_wave = AP && ap_chunk >= 0 && wave == ap_chunk % kWaves;
  uint16_t ax[4] = {0, 0, 0, 0};
  if (ap_wave) {
    const uint16_t *kx = p.k_new + static_cast<long>(unit) * D, *vx = p.v_new + static_cast<long>(unit) * D;
    ax[0] = kx[lane];
    ax[1] = kx[lane + 64];
    ax[2] = vx[lane];
    ax[3] = vx[lane + 64];
  }
  auto append = [&]() {
    const long row = cache_row(p.pg, unit, p.ap_offset, p.capacity);
    uint32_t *stage = lds + L::bmax;
    append_side(p.k, p.k_thr, p.sign, ax[0], ax[1], row, lane, stage);
    append_side(p.v, p.v_thr, p.sign, ax[2], ax[3], row, lane, stage);
  };
  if (ap_wave && ap_chunk < kWaves) {
    append();
    __builtin_amdgcn_s_waitcnt(0);  // the stores complete before the chunk is loaded
    asm volatile("" ::: "memory");
  }
  const bool ap_late = ap_wave && ap_chunk >= kWaves;
  ChunkData<KB, VB, GP> A, B;
  W.load(s0 + wave * kChunk, A);
  // The 16 (V) and up to 16 (K) centroids the tables need: every wave reads
  // them with uniform indices (scalar loads of the kernel arguments) into
  // its lanes 0-15, rather than one vector load of the argument block per
  // thread, and takes an entry's pair from those lanes with a shuffle.
  float kc = 0.0f, vc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (k_rot) kc = (lane == i) ? p.k_cent[i] : kc;
    if (KB != kInt8) vc = (lane == i) ? p.v_cent[i] : vc;
  }
  // Tables, written four replicas (16 bytes) at a time: the value table
  // (for KB = 4 also the K lo table, and the K hi table beside 3-bit V; for
  // KB = 3 also the K hi and lo tables).  Built while the query and the
  // first chunk are in flight.  Every loop below runs whole waves (the
  // counts are multiples of 64), as the shuffles need.
  constexpr int kVWord = v_table_byte<KB, VB>() / 4;
  for (int i = threadIdx.x; KB != kInt8 && i < 256 * (kRep / 4); i += kThreads) {
    const int e = i >> 3, r4 = 4 * (i & 7);
    const uint32_t w = VB == 4   ? pack_half2(__shfl(vc, e & 15), __shfl(vc, e >> 4))
                       : VB == 3 ? pack_half2(__shfl(vc, e & 7), __shfl(vc, (e >> 3) & 7))
                                 : pack_half2(__shfl(vc, e & 3), __shfl(vc, (e >> 2) & 3));
    *reinterpret_cast<u32x4_t *>(lds + kVWord + e * 64 + r4) = u32x4_t{w, w, w, w};
    if (KB) {
      uint32_t h, l;
      if (KB == 4) {
        split_pair(__shfl(kc, e & 15), __shfl(kc, e >> 4), h, l);
      } else if (KB == 3) {
        split_pair(__shfl(kc, e & 7), __shfl(kc, (e >> 3) & 7), h, l);
      } else {
        split_pair(__shfl(kc, e & 3), __shfl(kc, (e >> 2) & 3), h, l);
      }
      if (two_tables<KB, VB>()) *reinterpret_cast<u32x4_t *>(lds + e * 64 + r4) = u32x4_t{h, h, h, h};
      *reinterpret_cast<u32x4_t *>(lds + e * 64 + 32 + r4) = u32x4_t{l, l, l, l};
    }
  }
  // first use of the query after the tables, so the wait for it comes here
  asm volatile("" : "+v"(qa_raw), "+v"(qb_raw)::"memory");
  float qa = h2f(static_cast<uint16_t>(qa_raw));
  float qb = h2f(static_cast<uint16_t>(qb_raw));
  // rotate q in registers: H diag(s) q (unnormalised), butterflies at
  // stride 64 inside the lane and at strides 32 .. 1 across lanes
  // sign word of coordinates 4 j4 .. 4 j4 + 3 for the output stage (thread
  // j4 = threadIdx % 32 of each head), taken now, while the kernel
  // arguments are at hand, and kept in a register
  uint32_t out_sign;
  {
    const int wsel = (threadIdx.x & 31) >> 3;
    out_sign = wsel == 0 ? p.sign[0] : p.sign[1];
    out_sign = wsel == 2 ? p.sign[2] : out_sign;
    out_sign = wsel == 3 ? p.sign[3] : out_sign;
  }
  if (k_rot && wave < G) {
    // signs of coordinates lane and lane + 64 (uniform words, per-lane select)
    const uint32_t sa = lane < 32 ? p.sign[0] : p.sign[1];
    const uint32_t sb = lane < 32 ? p.sign[2] : p.sign[3];
    qa = ((sa >> (lane & 31)) & 1u) ? -qa : qa;
    qb = ((sb >> (lane & 31)) & 1u) ? -qb : qb;
    const float a = qa + qb, c = qa - qb;
    qa = a;
    qb = c;
    qa = xor_butterfly<32>(qa, lane);
    qb = xor_butterfly<32>(qb, lane);
    qa = xor_butterfly<16>(qa, lane);
    qb = xor_butterfly<16>(qb, lane);
    qa = xor_butterfly<8>(qa, lane);
    qb = xor_butterfly<8>(qb, lane);
    qa = xor_butterfly<4>(qa, lane);
    qb = xor_butterfly<4>(qb, lane);
    qa = xor_butterfly<2>(qa, lane);
    qb = xor_butterfly<2>(qb, lane);
    qa = xor_butterfly<1>(qa, lane);
    qb = xor_butterfly<1>(qb, lane);
  }
  // scaled query as fp16 hi/lo pair words: word j of head h holds
  // coordinates 2 j, 2 j + 1 (hi at [0, 64), lo at [64, 128) of the row).
  // Even lanes pair their qa with the odd neighbour's, odd lanes their qb
  // with the even neighbour's.
  // The head's B column is also scaled by a power of two 2^e that puts its
  // largest element in [128, 256): hi and lo then carry full precision
  // whatever the query's magnitude (fp16 ranges from 2^-24 to 65504), and
  // the scores are multiplied by the exact 2^-e (qinv).
  uint32_t *qhl = reinterpret_cast<uint32_t *>(qw);
  float *qinvs = reinterpret_cast<float *>(lds + L::qinv);
  if (wave < G) {
    const float qscale = k_rot ? kLog2e / static_cast<float>(D) : kLog2e / sqrtf(static_cast<float>(D));
    float amax = fmaxf(fabsf(qa), fabsf(qb));
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    amax *= qscale;
    int ex = 0;
    if (amax > 0.0f) (void)frexpf(amax, &ex);       // amax = f 2^ex, f in [0.5, 1)
    const float qs = ldexpf(qscale, 8 - ex);
    const float pa = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(qa), 0xb1, 0xf, 0xf, false));
    const float pb = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(qb), 0xb1, 0xf, 0xf, false));
    const bool odd = lane & 1;
    const float x0 = odd ? pb : qa, x1 = odd ? qb : pa;
    uint32_t h, l;
    split_pair(x0 * qs, x1 * qs, h, l);
    const int j = (odd ? 32 : 0) + (lane >> 1);
    qhl[wave * L::qstride + j] = h;
    qhl[wave * L::qstride + 64 + j] = l;
    if (lane == 0) qinvs[wave] = ldexpf(1.0f, ex - 8);
  } else if (wave < GP && lane == 0) {
    qinvs[wave] = 1.0f;
  }
  if (lane == 0) prog[wave] = 0;
  if (SP && threadIdx.x < 128) reinterpret_cast<float *>(lds + L::bmax)[threadIdx.x] = -INFINITY;
  __syncthreads();  // tables, rotated query and progress counters complete
  {
    // B operand of the score: column h < G the hi half of head h's query,
    // column GP + h its lo half, zero elsewhere; the MFMA then yields both
    // products, which the score adds (column h + GP into column h)
    const int hsel = W.col < GP ? W.col : W.col - GP;
    const bool live = W.col < 2 * GP && hsel < G;
    W.qinv = qinvs[W.col % GP];
    const uint32_t *row = qhl + (live ? hsel : 0) * L::qstride + (W.col < GP ? 0 : 64) + 16 * W.grp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // words 16 grp + 4 c .. + 3: coordinates 32 grp + 8 c .. + 7
      u32x4_t h = *reinterpret_cast<const u32x4_t *>(row + 4 * c);
      if (!live) h = u32x4_t{0u, 0u, 0u, 0u};
      W.bq[c] = __builtin_bit_cast(half8_t, h);
    }
  }

  if (ap_late) {
    // after the prologue, which it then does not delay; the stores complete
    // before the loop loads the position's chunk
    append();
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
  }

  // ---- main loop: the wave processes its chunk while its next one loads
  // into the other of two register buffers (ping-pong, so nothing is
  // copied).  Only the split's last chunk can be partial.
  Balance<kWaves, 4u * L::prog> bal;
  // sparse-V: after the first round of chunks (chunk c = wave), when every
  // wave has a full chunk in it, the waves exchange their running maxima at
  // one block barrier.  A decision from the other waves' maxima at any other
  // time would depend on how far they had got; this one is the same on
  // every call.  (More exchanges measured slower: each barrier waits for
  // the slowest wave.)
  // (chunk c = wave is always the first half of a loop iteration)
  auto exchange = [&](int cc) {
    if (cc == wave && kWaves <= n_full) W.exchange_max();
  };
  if (KB == 0) {
    // fp16 K rows (32 dwords a buffer): the masked variant stays inside the
    // loop, which keeps this shape within its registers
    int c = wave;
    const int last = max(n_chunks - 1, 0);
    uint32_t nblk = W.blk_fetch(s0 + min(c + kWaves, last) * kChunk);
    while (c < n_chunks) {
      int cn = c + kWaves;
      uint32_t nblk2 = W.blk_fetch(s0 + min(cn + kWaves, last) * kChunk);
      if (PG) asm volatile("" ::: "memory");
      W.load_row(W.row_from(nblk, s0 + min(cn, last) * kChunk), s0 + min(cn, last) * kChunk, B, SP && W.pred_skip);
      nblk = nblk2;
      asm volatile("" ::: "memory");
      if (c < n_full) {
        W.template cold_chunk<false, SP>(s0 + c * kChunk, s1, A, scores, hq0, p.length);
      } else {
        W.template cold_chunk<true, SP>(s0 + c * kChunk, s1, A, scores, hq0, p.length);
      }
      bal.step(wave, lane);
      if (SP) exchange(c);
      c = cn;
      if (c >= n_chunks) break;
      cn = c + kWaves;
      nblk2 = W.blk_fetch(s0 + min(cn + kWaves, last) * kChunk);
      if (PG) asm volatile("" ::: "memory");
      W.load_row(W.row_from(nblk, s0 + min(cn, last) * kChunk), s0 + min(cn, last) * kChunk, A, SP && W.pred_skip);
      nblk = nblk2;
      asm volatile("" ::: "memory");
      if (c < n_full) {
        W.template cold_chunk<false, SP>(s0 + c * kChunk, s1, B, scores, hq0, p.length);
      } else {
        W.template cold_chunk<true, SP>(s0 + c * kChunk, s1, B, scores, hq0, p.length);
      }
      bal.step(wave, lane);
      c = cn;
    }
  } else {
    // the loop body has no masking; a claimed partial chunk runs after it
    // The next chunk's loads are issued unconditionally (past the split
    // they re-read the last chunk, which the caches hold) and pinned before
    // the current chunk's work, so the compiler cannot sink them.
    int c = wave;
    bool in_b = false;  // the buffer holding chunk c
    const int last = max(n_chunks - 1, 0);
    // Paged: the table entry of the chunk loaded next is fetched one load
    // ahead, before the loads it runs ahead of, so waiting for it never
    // waits for a chunk still needed later.
    uint32_t nblk = W.blk_fetch(s0 + min(c + kWaves, last) * kChunk);
    while (c < n_full) {
      int cn = c + kWaves;
      uint32_t nblk2 = W.blk_fetch(s0 + min(cn + kWaves, last) * kChunk);
      if (PG) asm volatile("" ::: "memory");
      W.load_row(W.row_from(nblk, s0 + min(cn, last) * kChunk), s0 + min(cn, last) * kChunk, B, SP && W.pred_skip);
      nblk = nblk2;
      asm volatile("" ::: "memory");
      W.template cold_chunk<false, SP>(s0 + c * kChunk, s1, A, scores, hq0, p.length);
      bal.step(wave, lane);
      if (SP) exchange(c);
      c = cn;
      if (c >= n_full) {
        in_b = true;
        break;
      }
      cn = c + kWaves;
      nblk2 = W.blk_fetch(s0 + min(cn + kWaves, last) * kChunk);
      if (PG) asm volatile("" ::: "memory");
      W.load_row(W.row_from(nblk, s0 + min(cn, last) * kChunk), s0 + min(cn, last) * kChunk, A, SP && W.pred_skip);
      nblk = nblk2;
      asm volatile("" ::: "memory");
      W.template cold_chunk<false, SP>(s0 + c * kChunk, s1, B, scores, hq0, p.length);
      // (balanced once per two chunks here: measured faster for these shapes)
      c = cn;
    }
    if (c < n_chunks) {
      if (in_b) {
        W.template cold_chunk<true, SP>(s0 + c * kChunk, s1, B, scores, hq0, p.length);
      } else {
        W.template cold_chunk<true, SP>(s0 + c * kChunk, s1, A, scores, hq0, p.length);
      }
    }
  }

  // ---- merge the waves of this block (tables are dead from here on) -----
  __builtin_amdgcn_s_setprio(0);
  if (!L::own_slots) __syncthreads();  // the slots overlay the tables
  W.to_slot(slots + wave * GP * kPS, false);
  __syncthreads();
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + p.ws_part_off);
  float *mypart = part + (static_cast<long>(vunit) * nsplit + split) * Gs * kPS;
  if (threadIdx.x < G * (D / 4)) {
    // thread (h, j4): head h, values 4 j4 .. 4 j4 + 3, L2-coherent stores
    const int h = threadIdx.x / (D / 4), j4 = threadIdx.x % (D / 4);
    float4 hdr, val;
    merge_slots<kWaves, GP>(slots, h, j4, hdr, val);
    const auto rs = rsrc(mypart, G * kPS * 4);
    if (j4 == 0) store4_coherent(rs, h * kPS * 4, hdr);
    store4_coherent(rs, (h * kPS + kPV + 4 * j4) * 4, val);
  }

  // ---- the last block of the unit merges the splits ----------------------
  // The partials above are L2-coherent stores; once they have completed
  // (s_waitcnt), the arrival counter is bumped.  The last arrival reads all
  // partials with L2-coherent loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(p.counters + vunit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == static_cast<unsigned>(nsplit - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;

  // delegated V: this block also attends over the fp16 hot window
  float *hotp = work + kWaves * GP * kPS;  // [G][kPS] merged hot partial
  const int h0 = p.cold_len, h1 = p.length;
  const bool has_hot = h1 > h0;
  if (has_hot) {
    // the window's chunks on the 32-position grid from floor(h0 / 32) 32,
    // dealt to the waves in equal runs; positions below h0 are masked
    const int c0 = h0 / kChunk * kChunk;
    const int hspan = h1 - c0;
    const int hper = ((hspan + kWaves - 1) / kWaves + kChunk - 1) / kChunk * kChunk;
    const int hs = c0 + wave * hper, he = min(h1, hs + hper);
    W.reset();
    W.vscale = 1.0f;
    for (int t0 = hs; t0 < he; t0 += kChunk) {
      W.load(t0, A);
      W.hot_chunk(t0, h0, he, A, scores, hq0, p.length);
    }
    W.to_slot(work + wave * GP * kPS, true);
    __syncthreads();
    if (threadIdx.x < G * (D / 4)) {
      const int h = threadIdx.x / (D / 4), j4 = threadIdx.x % (D / 4);
      float4 hdr, val;
      merge_slots<kWaves, GP>(work, h, j4, hdr, val);
      if (j4 == 0) *reinterpret_cast<float4 *>(hotp + h * kPS) = hdr;
      *reinterpret_cast<float4 *>(hotp + h * kPS + kPV + 4 * j4) = val;
    }
    __syncthreads();
  }
  // Every load below is independent of the others, so each thread has all of
  // its partial results in flight at once.  Thread (h, j4) owns head h,
  // coordinates 4 j4 .. 4 j4 + 3; the 32 threads of a head sit in one wave,
  // so the inverse rotation needs no block barrier.
  if (threadIdx.x >= G * (D / 4)) return;
  const float *up = part + static_cast<long>(vunit) * nsplit * Gs * kPS;
  const int hh = threadIdx.x / (D / 4);
  const int jj = 4 * (threadIdx.x % (D / 4));
  float *orow = p.out + (hq0 + hh) * D + jj;
  float r4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, q4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float Lt = 0.0f;
  float M = -INFINITY;
  // partials of the unit, read past the non-coherent caches (sc1)
  const auto rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(up), 0, nsplit * Gs * kPS * 4, 0x00020000);
  constexpr int kB = 8;  // splits per batch of independent loads
  for (int sp0 = 0; sp0 < nsplit; sp0 += kB) {
    float mv[kB], lv[kB], ov[kB][4];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int sp = min(sp0 + k, nsplit - 1);
      const int base = ((sp * Gs + hh) * kPS) * 4;
      const u32x2_t ml = __builtin_amdgcn_raw_buffer_load_b64(rp, base, 0, kCoherentLoad);
      const u32x4_t o4 = __builtin_amdgcn_raw_buffer_load_b128(rp, base + (kPV + jj) * 4, 0, kCoherentLoad);
      mv[k] = (sp0 + k < nsplit) ? __uint_as_float(ml[0]) : -INFINITY;
      lv[k] = __uint_as_float(ml[1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[k][e] = __uint_as_float(o4[e]);
    }
    float mg = M;
#pragma unroll
    for (int k = 0; k < kB; ++k) mg = fmaxf(mg, mv[k]);
    if (mg == -INFINITY) continue;
    const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - mg);
    M = mg;
    Lt *= a;
#pragma unroll
    for (int e = 0; e < 4; ++e) r4[e] *= a;
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const float w = (mv[k] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv[k] - M);
      Lt += w * lv[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) r4[e] += w * ov[k][e];
    }
  }
  if (has_hot) {
    const float mh = hotp[hh * kPS];
    if (mh != -INFINITY) {
      const float mg = fmaxf(M, mh);
      const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - mg);
      const float bh = __builtin_amdgcn_exp2f(mh - mg);
      Lt = Lt * a + bh * hotp[hh * kPS + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r4[e] *= a;
        q4[e] = bh * hotp[hh * kPS + kPV + jj + e];
      }
    }
  }
  float4 o;
  const float inv = (Lt > 0.0f) ? __builtin_amdgcn_rcpf(Lt) : 0.0f;  // within 1 ulp
  if (KB == kInt8) {
    // original domain; the value operands were x 2^-10
    o.x = r4[0] * 1024.0f * inv;
    o.y = r4[1] * 1024.0f * inv;
    o.z = r4[2] * 1024.0f * inv;
    o.w = r4[3] * 1024.0f * inv;
    *reinterpret_cast<float4 *>(orow) = o;
    if (threadIdx.x == 0) __hip_atomic_store(p.counters + vunit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // inverse rotation diag(s) H / sqrt(d): butterflies at strides 1 and 2
  // inside the thread, strides 4 .. 64 across the head's 32 lanes
  {
    const float b0 = r4[0] + r4[1], b1 = r4[0] - r4[1], b2 = r4[2] + r4[3], b3 = r4[2] - r4[3];
    r4[0] = b0 + b2;
    r4[1] = b1 + b3;
    r4[2] = b0 - b2;
    r4[3] = b1 - b3;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r4[e] = xor_butterfly<1>(r4[e], lane);
    r4[e] = xor_butterfly<2>(r4[e], lane);
    r4[e] = xor_butterfly<4>(r4[e], lane);
    r4[e] = xor_butterfly<8>(r4[e], lane);
    r4[e] = xor_butterfly<16>(r4[e], lane);
  }
  const float rs = 1.0f / sqrtf(static_cast<float>(D));
  const uint32_t sbits = out_sign >> (jj & 31);
  o.x = ((sbits & 1u) ? -r4[0] : r4[0]) * rs;
  o.y = ((sbits & 2u) ? -r4[1] : r4[1]) * rs;
  o.z = ((sbits & 4u) ? -r4[2] : r4[2]) * rs;
  o.w = ((sbits & 8u) ? -r4[3] : r4[3]) * rs;
  o.x = (o.x + q4[0]) * inv;
  o.y = (o.y + q4[1]) * inv;
  o.z = (o.z + q4[2]) * inv;
  o.w = (o.w + q4[3]) * inv;
  *reinterpret_cast<float4 *>(orow) = o;
  if (threadIdx.x == 0) __hip_atomic_store(p.counters + vunit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

template <int KB, int VB, int GP, bool SC, bool SP, bool AP = false>
void launch_sp(const DecodeParams &p, dim3 grid, hipStream_t stream) {
  if (p.pg.table) {
    hipLaunchKernelGGL((decode_mfma_kernel<KB, VB, GP, true, SC, SP, AP>), grid, dim3(64 * waves_of<KB>()), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<KB, VB, GP, false, SC, SP, AP>), grid, dim3(64 * waves_of<KB>()), 0, stream, p);
  }
}

// SP: sparse-V (a threshold is set); the exact decode compiles it out
template <int KB, int VB, int GP, bool SC>
void launch_sc(const DecodeParams &p, dim3 grid, hipStream_t stream) {
  if (p.sparse_lg != -INFINITY) {
    launch_sp<KB, VB, GP, SC, true>(p, grid, stream);
  } else {
    launch_sp<KB, VB, GP, SC, false>(p, grid, stream);
  }
}

template <int KB, int VB, int GP>
void launch_gp(const DecodeParams &p, dim3 grid, hipStream_t stream) {
  if (p.ap_split >= 0) {
    // fused append: exact decode, no scores (the host checks both; delegated
    // sides take the two separate calls instead)
    launch_sp<KB, VB, GP, false, false, true>(p, grid, stream);
    return;
  }
  if (p.scores) {
    launch_sc<KB, VB, GP, true>(p, grid, stream);
  } else {
    launch_sc<KB, VB, GP, false>(p, grid, stream);
  }
}

template <int KB, int VB>
void launch_kb(const DecodeParams &p, dim3 grid, hipStream_t stream) {
  const int G = p.q_heads / p.kv_heads;
  if (G <= 4) {
    launch_gp<KB, VB, 4>(p, grid, stream);
  } else {
    launch_gp<KB, VB, 8>(p, grid, stream);
  }
}

hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t stream) {
  const int G = p.q_heads / p.kv_heads;
  const int kb = p.k.mode == TQ_SIDE_PACKED ? p.k.bits : (p.k.mode == TQ_SIDE_INT8 ? kInt8 : 0);
  if ((kb == kInt8) != (p.v.mode == TQ_SIDE_INT8)) return hipErrorInvalidValue;
  if (G < 1 || p.head_dim != D) return hipErrorInvalidValue;
  // head groups of at most 8 query heads, each a unit with its own counter
  const long vunits = static_cast<long>(p.batch) * p.kv_heads * ((G + 7) / 8);
  if (vunits > kMfmaMaxUnits) return hipErrorInvalidValue;
  const int nsplit = p.n_cold_splits;
  if (nsplit < 1 || nsplit > kMaxSplits || p.n_hot_splits != 0) return hipErrorInvalidValue;
  // every split starts on the chunk grid (a paged chunk lies in one block)
  if (p.cold_split_len < 1 || p.cold_split_len % kChunk) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(vunits * nsplit));
  if (kb == kInt8) {
    launch_kb<kInt8, kInt8>(p, grid, stream);
    return hipGetLastError();
  }
  // packed or delegated V at 2, 3 or 4 bits; 4-bit K beside 4-bit V reads
  // the V table for its hi half, so it needs the same codebook
  const int vb = p.v.bits;
  if (kb == 4 && vb == 4 && !p.share_lut) return hipErrorInvalidValue;
  switch (kb * 16 + vb) {
    case 2: launch_kb<0, 2>(p, grid, stream); break;
    case 3: launch_kb<0, 3>(p, grid, stream); break;
    case 4: launch_kb<0, 4>(p, grid, stream); break;
    case 2 * 16 + 2: launch_kb<2, 2>(p, grid, stream); break;
    case 2 * 16 + 3: launch_kb<2, 3>(p, grid, stream); break;
    case 3 * 16 + 3: launch_kb<3, 3>(p, grid, stream); break;
    case 3 * 16 + 4: launch_kb<3, 4>(p, grid, stream); break;
    case 4 * 16 + 3: launch_kb<4, 3>(p, grid, stream); break;
    case 4 * 16 + 4: launch_kb<4, 4>(p, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq
