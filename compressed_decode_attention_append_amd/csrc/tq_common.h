// Shared host/device definitions of libtq: kernel parameter blocks and the
// launchers each kernel file provides.  Internal; the public ABI is tq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kMaxLevels = 1 << TQ_MAX_BITS;   // 256 centroids, 255 thresholds
constexpr int kMaxSignWords = TQ_MAX_HEAD_DIM / 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device view of one side of a cache.
struct SideDev {
  int mode;        // TQ_SIDE_*
  int bits;        // code width (packed / delegated)
  int words;       // uint32 words per packed row
  int hot;         // delegated ring length
  uint32_t *codes; // [B][H][cap][words]
  float *norms;    // [B][H][cap]
  uint16_t *fp16;  // fp16 rows (FP16) or hot ring (DELEGATED)
};

// Where a cache row lives.  Contiguous (table null): row (b Hkv + kv) cap
// + t.  Paged: row (table[b][t / bs] Hkv + kv) bs + t % bs of the block
// pools.  `bh` is b Hkv + kv.
struct Paging {
  const int32_t *table;  // [B][max_blocks] or null
  int bs, max_blocks, kv_heads;
  int num_blocks;        // blocks in each pool: table entries in [0, num_blocks) are valid
};

// Block index a table entry names, or -1 when the entry lies outside the
// pools (such a block reads as zero rows and takes no writes).
__host__ __device__ inline long valid_block(const Paging &pg, int entry) {
  return static_cast<unsigned>(entry) < static_cast<unsigned>(pg.num_blocks) ? static_cast<long>(entry) : -1L;
}

// Paged row of position t of (sequence b, KV head kv), or -1 in an
// out-of-range block.  Unsigned 32-bit arithmetic for the divisions:
// positions and bh = b Hkv + kv (at most 65535) fit, and a 64-bit division
// costs tens of instructions.
__host__ __device__ inline long paged_row(const Paging &pg, int b, int kv, int t) {
  const unsigned ut = static_cast<unsigned>(t), ubs = static_cast<unsigned>(pg.bs);
  const unsigned blk = ut / ubs;
  const long e = valid_block(pg, pg.table[b * pg.max_blocks + static_cast<int>(blk)]);
  return e < 0 ? -1L : (e * pg.kv_heads + kv) * pg.bs + static_cast<int>(ut - blk * ubs);
}

// Storage row of position t of unit bh; -1 in an out-of-range block.
__host__ __device__ inline long cache_row(const Paging &pg, long bh, int t, int capacity) {
  if (!pg.table) return bh * capacity + t;
  const unsigned u = static_cast<unsigned>(bh), kvh = static_cast<unsigned>(pg.kv_heads);
  const unsigned b = u / kvh;
  return paged_row(pg, static_cast<int>(b), static_cast<int>(u - b * kvh), t);
}

struct QuantizeParams {
  SideDev k, v;
  const uint16_t *k_new;  // [B][H][n_new][d] fp16
  const uint16_t *v_new;
  int batch, heads, head_dim, capacity, n_new, offset;
  Paging pg;
  int side_mask;                 // sides this launch encodes: bit 0 K, bit 1 V
  float k_lut_scale;             // matrix-core kernel: code-table cells per unit of y
  float v_lut_scale;             //   (a power of two; 0 = side not eligible)
  uint32_t sign[kMaxSignWords];  // bit j set: s_j = -1
  float k_thr[kMaxLevels];       // thresholds (L-1 used)
  float v_thr[kMaxLevels];
};

struct DequantParams {
  SideDev s;
  float *out;  // [B][H][count][d]
  int batch, heads, head_dim, capacity, start, count;
  Paging pg;
  uint32_t sign[kMaxSignWords];
  float cent[kMaxLevels];
};

struct DecodeParams {
  SideDev k, v;
  const uint16_t *q;  // [B][Hq][d] fp16
  float *out;         // [B][Hq][d]
  float *scores;      // [B][Hq][length] or null
  float *ws;          // workspace base
  unsigned *counters; // per-unit arrival counters (start of the workspace)
  size_t ws_part_off; // byte offset of the partial results
  int batch, kv_heads, q_heads, head_dim, capacity, length;
  Paging pg;
  // sparse-V: log2 of the weight threshold below which a group's values may
  // be skipped; -inf = exact
  float sparse_lg;
  // plain split-context variant
  int n_splits, split_len;
  // matrix-core variant: packed (cold) positions [0, cold_len) in
  // n_cold_splits splits, fp16 hot positions [cold_len, length) in
  // n_hot_splits splits
  int cold_len, n_cold_splits, cold_split_len, n_hot_splits, hot_split_len;
  int share_lut;      // K and V use the same 4-bit codebook
  uint32_t sign[kMaxSignWords];
  float k_cent[kMaxLevels];
  float v_cent[kMaxLevels];
  // fused append (matrix-core kernel): the new rows k_new / v_new (fp16
  // [B][Hkv][1][d]) are written at position ap_offset by the blocks of split
  // ap_split before they read them; ap_split = -1: nothing is appended.
  const uint16_t *k_new, *v_new;
  int ap_offset, ap_split;
  float k_thr[16], v_thr[16];  // packed sides' thresholds (at most 4 bits here)
};

// Workspace: a fixed region of per-unit counters (zero on entry, left zero
// on exit), then the partial results of whichever variant runs.
constexpr size_t kCounterBytes = size_t(65536) * sizeof(unsigned);
static_assert(kCounterBytes == TQ_WORKSPACE_COUNTER_BYTES, "tq.h states the counter region's size");

// Plain variant's partials (floats, each region 256-byte aligned):
//   ml   [B*Hq][n_splits][2]   running max (log2 domain) and sum
//   orot [B*Hq][n_splits][d]   rotated-domain value accumulator (packed V)
//   ohot [B*Hq][n_splits][d]   original-domain accumulator (fp16 V rows)
struct DecodeWorkspace {
  size_t ml_off, orot_off, ohot_off, total;  // in bytes
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline DecodeWorkspace decode_workspace_layout(int batch, int q_heads,
                                                                   int n_splits, int head_dim) {
  DecodeWorkspace w;
  const size_t units = size_t(batch) * q_heads * n_splits;
  w.ml_off = kCounterBytes;
  w.orot_off = w.ml_off + align256(units * 2 * sizeof(float));
  w.ohot_off = w.orot_off + align256(units * head_dim * sizeof(float));
  w.total = w.ohot_off + align256(units * head_dim * sizeof(float));
  return w;
}

// Matrix-core variant's partials: [B*Hkv][splits][G][d + 2] floats holding
// (max, sum, accumulator[d]) per query head.
// A query group of G > 8 heads runs as ceil(G / 8) head groups of at most 8,
// each with partials for 8 heads.
inline size_t decode_mfma_workspace_bytes(int batch, int kv_heads, int q_heads, int splits,
                                          int head_dim) {
  const size_t G = size_t(q_heads / kv_heads);
  const size_t groups = (G + 7) / 8, per = G < 8 ? G : 8;
  return kCounterBytes + align256(size_t(batch) * kv_heads * groups * splits * per * (head_dim + 4) * sizeof(float));
}

hipError_t launch_quantize_append(const QuantizeParams &p, hipStream_t stream);
// Matrix-core encoder for packed sides at head_dim 128 and 1..4 bits; the
// sides it takes are those with a non-zero lut scale in `p` and bit set in
// p.side_mask.
hipError_t launch_quantize_mfma(const QuantizeParams &p, hipStream_t stream);
// Power-of-two code-table scale for the matrix-core encoder (0 when the
// thresholds are too close for a scale of at most kQuantLutMaxScale; such a
// side goes to the plain encoder).  The Lloyd-Max codebooks at head_dim 128
// need 1, 16, 32 and 64 for 1..4 bits (smallest threshold gaps 2, 0.087,
// 0.044, 0.023), so the table holds at most 131 cells a side and leaves the
// LDS to the kernel's occupancy.
float quantize_lut_scale(const float *thr, int bits);
constexpr int kQuantLutMaxScale = 64;
hipError_t launch_dequantize(const DequantParams &p, hipStream_t stream);
hipError_t launch_read_probe(const void *buf, size_t bytes, unsigned *sink, hipStream_t stream);
// Zero `bytes` (a multiple of 16) of device memory at a 16-byte aligned `buf`.
hipError_t launch_zero_fill(void *buf, size_t bytes, hipStream_t stream);
// Size of the fixed per-device decode scratch (tq_decode_attention_noalloc),
// and its device address on the device `stream` runs on (set up on first use).
constexpr size_t kScratchBytes = size_t(16) << 20;
static_assert(kScratchBytes == TQ_NOALLOC_SCRATCH_BYTES, "tq.h states the scratch size");
hipError_t scratch_workspace(hipStream_t stream, void **ptr);
hipError_t launch_decode_ref(const DecodeParams &p, hipStream_t stream);
// The matrix-core decode takes head_dim 128, any number of query heads per
// KV head (more than 8 as head groups of at most 8, at most kMfmaMaxUnits
// (batch, KV head, head group) units), and either INT8 on both sides, or a
// packed or delegated V of 2 to 4 bits with fp16 K, or packed K and V as
// 2/2, 2/3, 3/3, 3/4, 4/3 bits, or 4/4 with one codebook; at most
// kMfmaMaxSplits context splits per unit, each a multiple of kMfmaChunk
// positions long.
// (The host picks it by this rule; the launcher checks it again.)
hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t stream);
constexpr int kMfmaMaxSplits = 256;
constexpr long kMfmaMaxUnits = long(kCounterBytes / sizeof(unsigned));  // one arrival counter each
constexpr int kMfmaChunk = 32;  // positions the matrix-core decode reads as one chunk

}  // namespace tq
