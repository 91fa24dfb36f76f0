// C ABI of libtq: argument validation, rotation signs, parameter blocks and
// kernel dispatch.  Every check runs on the host before any HIP call, so an
// invalid call launches nothing and writes nothing.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "tq.h"
#include "tq_common.h"

namespace {

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

int words_of(int d, int bits) { return (bits * d + 31) / 32; }

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): add the golden-ratio
// increment to the state, then two xor-shift-multiply rounds and a final
// xor-shift give the output.
uint64_t splitmix64_next(uint64_t &state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void fill_signs(uint64_t seed, int d, uint32_t *words) {
  uint64_t state = seed;
  for (int w = 0; w < tq::kMaxSignWords; ++w) words[w] = 0;
  for (int j = 0; j < d; ++j) {
    if (splitmix64_next(state) >> 63) words[j >> 5] |= 1u << (j & 31);
  }
}

int check_side(const tq_side &s, bool is_v) {
  switch (s.mode) {
    case TQ_SIDE_FP16:
      return s.fp16 ? TQ_OK : TQ_ERR_ARG;
    case TQ_SIDE_INT8:
      return (s.codes && s.norms) ? TQ_OK : TQ_ERR_ARG;
    case TQ_SIDE_PACKED:
    case TQ_SIDE_DELEGATED:
      if (s.mode == TQ_SIDE_DELEGATED && !is_v) return TQ_ERR_MODE;
      if (s.bits < TQ_MIN_BITS || s.bits > TQ_MAX_BITS) return TQ_ERR_BITS;
      if (!s.codes || !s.norms || !s.centroids || !s.thresholds) return TQ_ERR_ARG;
      if (s.mode == TQ_SIDE_DELEGATED && (s.hot < 1 || !s.fp16)) return TQ_ERR_ARG;
      return TQ_OK;
    default:
      return TQ_ERR_MODE;
  }
}

int check_cache(const tq_cache *c) {
  if (!c) return TQ_ERR_ARG;
  if (!head_dim_ok(c->head_dim)) return TQ_ERR_HEAD_DIM;
  if (c->batch < 1 || c->kv_heads < 1 || c->capacity < 0) return TQ_ERR_ARG;
  if (static_cast<long long>(c->batch) * c->kv_heads > 65535) return TQ_ERR_ARG;
  if (c->block_table) {
    // paged: whole 32-position chunks per block, and the table covers the
    // capacity exactly
    if (c->block_size < 32 || c->block_size % 32 || c->max_blocks < 1 || c->num_blocks < 1) return TQ_ERR_ARG;
    if (static_cast<long long>(c->block_size) * c->max_blocks != c->capacity) return TQ_ERR_ARG;
  }
  int r = check_side(c->k, false);
  if (r != TQ_OK) return r;
  return check_side(c->v, true);
}

tq::Paging paging_of(const tq_cache *c) {
  tq::Paging pg;
  pg.table = c->block_table;
  pg.bs = c->block_table ? c->block_size : 0;
  pg.max_blocks = c->block_table ? c->max_blocks : 0;
  pg.kv_heads = c->kv_heads;
  pg.num_blocks = c->block_table ? c->num_blocks : 0;
  return pg;
}

tq::SideDev side_dev(const tq_side &s, int d) {
  tq::SideDev o;
  o.mode = s.mode;
  o.bits = (s.mode == TQ_SIDE_FP16) ? 0 : (s.mode == TQ_SIDE_INT8 ? 8 : s.bits);
  o.words = (s.mode == TQ_SIDE_FP16) ? 0 : words_of(d, o.bits);
  o.hot = s.hot;
  o.codes = s.codes;
  o.norms = s.norms;
  o.fp16 = s.fp16;
  return o;
}

// Codebook levels of a side: 2^bits for the TurboQuant modes, none for fp16
// and INT8 sides (whose bit field is not read).
int n_levels(const tq_side &s) {
  return (s.mode == TQ_SIDE_PACKED || s.mode == TQ_SIDE_DELEGATED) ? (1 << s.bits) : 0;
}

void copy_levels(const tq_side &s, const float *src, int n, float *dst) {
  for (int i = 0; i < tq::kMaxLevels; ++i) dst[i] = 0.0f;
  if ((s.mode == TQ_SIDE_PACKED || s.mode == TQ_SIDE_DELEGATED) && src) memcpy(dst, src, sizeof(float) * n);
}

// Context split of the plain decode.  A block walks its range in tiles of 32
// or 64 positions for up to eight query heads; the automatic split aims at
// about 1024 blocks (four per compute unit, one round at the kernel's usual
// occupancy) in multiples of 32 positions.  Any split length fits the
// block's LDS.
bool choose_split(const tq_cache *c, int q_heads, int length, int n_splits, int *ns, int *sl) {
  constexpr long kTargetBlocks = 1024;
  constexpr int kTile = 32;
  const int G = q_heads / c->kv_heads;
  int split;
  if (n_splits > 0) {
    split = length > 0 ? (length + n_splits - 1) / n_splits : 1;
    *ns = n_splits;
  } else {
    const long per_split = static_cast<long>(c->batch) * c->kv_heads * ((G + 7) / 8);
    const long want = (static_cast<long>(length) * per_split + kTargetBlocks - 1) / kTargetBlocks;
    split = static_cast<int>(std::max<long>(kTile, (want + kTile - 1) / kTile * kTile));
    *ns = length > 0 ? (length + split - 1) / split : 1;
  }
  *sl = std::max(split, 1);
  return true;
}

// Which decode runs: the matrix-core kernel when it supports the shape,
// else the plain one.  TQ_DECODE_VARIANT=ref forces the plain kernel (A/B
// measurements and the cross-check tests).
enum Variant { kRef, kMfma };

// The shapes the matrix-core decode takes (tq_common.h states the rule).
bool decode_mfma_supported(const tq::DecodeParams &p) {
  const int G = p.q_heads / p.kv_heads;
  if (p.head_dim != 128) return false;
  // more than 8 query heads a KV head: head groups of 8, one counter each
  if (static_cast<long>(p.batch) * p.kv_heads * ((G + 7) / 8) > tq::kMfmaMaxUnits) return false;
  if (p.k.mode == TQ_SIDE_INT8 || p.v.mode == TQ_SIDE_INT8) return p.k.mode == p.v.mode;  // INT8 on both sides
  if (!(p.v.mode == TQ_SIDE_PACKED || p.v.mode == TQ_SIDE_DELEGATED) || p.v.bits < 2 || p.v.bits > 4) return false;
  if (p.k.mode == TQ_SIDE_FP16) return true;
  if (p.k.mode != TQ_SIDE_PACKED || p.v.mode != TQ_SIDE_PACKED) return false;
  // the floor/ceil splits of 2 to 4 bits, and 4-bit K beside 3-bit V; 4-bit
  // K beside 4-bit V shares V's codebook table
  const int kb = p.k.bits, vb = p.v.bits;
  return (kb == 2 && vb <= 3) || (kb == 3 && vb >= 3) || (kb == 4 && (vb == 3 || (vb == 4 && p.share_lut)));
}

Variant pick_variant(const tq::DecodeParams &p) {
  const char *env = getenv("TQ_DECODE_VARIANT");
  if (env && strcmp(env, "ref") == 0) return kRef;
  return decode_mfma_supported(p) ? kMfma : kRef;
}

// Splits of the matrix-core kernel: the packed positions of a unit in
// n_cold splits of a multiple of 256 positions (8 waves x 32), aiming at one
// block per compute unit (256 blocks) with at least 512 positions per block.
// An explicit split count still gives splits of a multiple of 32 positions:
// the kernel reads 32-position chunks from each split's start, and a paged
// chunk must lie in one block (blocks are multiples of 32 positions), so
// every split starts on that grid.  The fp16 hot window of a delegated V is
// attended by the block that finishes its unit last, so it needs no split
// of its own.
void mfma_splits(const tq_cache *c, int length, int n_splits, tq::DecodeParams *p) {
  constexpr int kTargetBlocks = 256, kMinPerBlock = 512, kQuantum = 256;
  const int units = c->batch * c->kv_heads * ((p->q_heads / c->kv_heads + 7) / 8);
  const int cold = (c->v.mode == TQ_SIDE_DELEGATED) ? std::max(0, length - c->v.hot) : length;
  const int cap = tq::kMfmaMaxSplits;
  int ncold = 1, clen = tq::kMfmaChunk;
  if (cold > 0) {
    if (n_splits > 0) {
      ncold = std::min(std::min(n_splits, cold), cap);
      clen = ((cold + ncold - 1) / ncold + tq::kMfmaChunk - 1) / tq::kMfmaChunk * tq::kMfmaChunk;
    } else {
      const int want = std::max(1, std::min(std::min((kTargetBlocks + units - 1) / units,
                                                     (cold + kMinPerBlock - 1) / kMinPerBlock),
                                            cap));
      clen = ((cold + want - 1) / want + kQuantum - 1) / kQuantum * kQuantum;
    }
    ncold = (cold + clen - 1) / clen;
  }
  // an empty packed range still takes one split: it writes an empty partial
  // and, as the unit's last block, the hot window or the zero output
  p->cold_len = cold;
  p->n_cold_splits = ncold;
  p->cold_split_len = clen;
  p->n_hot_splits = 0;
  p->hot_split_len = length - cold;
}

void fill_decode_params(const tq_cache *cache, const void *q, int q_heads, int length,
                        tq::DecodeParams *p) {
  memset(p, 0, sizeof(*p));
  const int d = cache->head_dim;
  p->k = side_dev(cache->k, d);
  p->v = side_dev(cache->v, d);
  p->q = static_cast<const uint16_t *>(q);
  p->batch = cache->batch;
  p->kv_heads = cache->kv_heads;
  p->q_heads = q_heads;
  p->head_dim = d;
  p->capacity = cache->capacity;
  p->length = length;
  p->pg = paging_of(cache);
  fill_signs(cache->seed, d, p->sign);
  copy_levels(cache->k, cache->k.centroids, n_levels(cache->k), p->k_cent);
  copy_levels(cache->v, cache->v.centroids, n_levels(cache->v), p->v_cent);
  p->ap_split = -1;  // nothing appended (tq_decode_attention_append sets it)
  p->share_lut = (cache->k.mode == TQ_SIDE_PACKED && cache->k.bits == 4 && cache->v.bits == 4 &&
                  memcmp(p->k_cent, p->v_cent, sizeof(float) * 16) == 0)
                     ? 1
                     : 0;
}

// Workspace bytes the chosen variant needs (0 if the shape is invalid).
size_t workspace_need(const tq_cache *cache, int q_heads, int length, int n_splits,
                      tq::DecodeParams *p, Variant *v) {
  fill_decode_params(cache, reinterpret_cast<const void *>(1), q_heads, length, p);
  *v = pick_variant(*p);
  if (*v == kMfma) {
    mfma_splits(cache, length, n_splits, p);
    return tq::decode_mfma_workspace_bytes(cache->batch, cache->kv_heads, q_heads, p->n_cold_splits,
                                           cache->head_dim);
  }
  int ns = 0, sl = 0;
  if (!choose_split(cache, q_heads, length, n_splits, &ns, &sl)) return 0;
  p->n_splits = ns;
  p->split_len = sl;
  return tq::decode_workspace_layout(cache->batch, q_heads, ns, cache->head_dim).total;
}

}  // namespace

extern "C" {

const char *tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_ARG: return "invalid argument";
    case TQ_ERR_HEAD_DIM: return "head_dim must be a power of two in [32, 256]";
    case TQ_ERR_BITS: return "bits must be in [1, 8]";
    case TQ_ERR_CAPACITY: return "rows outside the cache capacity";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ_ERR_MODE: return "unsupported side mode";
    case TQ_ERR_HIP: return "HIP launch error";
    case TQ_ERR_SCRATCH: return "the decode needs more than the fixed 16 MiB scratch";
    default: return "unknown status";
  }
}

int tq_split_bits(double bits, int *k_bits, int *v_bits) {
  if (!k_bits || !v_bits) return TQ_ERR_ARG;
  if (!(bits == bits)) return TQ_ERR_BITS;
  const double lo = floor(bits), hi = ceil(bits);
  if (lo < TQ_MIN_BITS || hi > TQ_MAX_BITS) return TQ_ERR_BITS;
  *k_bits = static_cast<int>(lo);
  *v_bits = static_cast<int>(hi);
  return TQ_OK;
}

int tq_row_words(int head_dim, int bits) {
  if (!head_dim_ok(head_dim)) return TQ_ERR_HEAD_DIM;
  if (bits < TQ_MIN_BITS || bits > TQ_MAX_BITS) return TQ_ERR_BITS;
  return words_of(head_dim, bits);
}

int tq_sign_words(uint64_t seed, int head_dim, uint32_t *sign_words) {
  if (!sign_words) return TQ_ERR_ARG;
  if (!head_dim_ok(head_dim)) return TQ_ERR_HEAD_DIM;
  uint32_t w[tq::kMaxSignWords];
  fill_signs(seed, head_dim, w);
  memcpy(sign_words, w, sizeof(uint32_t) * (head_dim / 32));
  return TQ_OK;
}

int tq_quantize_append(const tq_cache *cache, const void *k_new, const void *v_new, int n_new,
                       int offset, void *hip_stream) {
  int r = check_cache(cache);
  if (r != TQ_OK) return r;
  if (n_new < 0) return TQ_ERR_ARG;
  if (offset < 0 || static_cast<long long>(offset) + n_new > cache->capacity) return TQ_ERR_CAPACITY;
  if (n_new == 0) return TQ_OK;
  if (!k_new || !v_new) return TQ_ERR_ARG;

  tq::QuantizeParams p;
  memset(&p, 0, sizeof(p));
  const int d = cache->head_dim;
  p.k = side_dev(cache->k, d);
  p.v = side_dev(cache->v, d);
  p.k_new = static_cast<const uint16_t *>(k_new);
  p.v_new = static_cast<const uint16_t *>(v_new);
  p.batch = cache->batch;
  p.heads = cache->kv_heads;
  p.head_dim = d;
  p.capacity = cache->capacity;
  p.n_new = n_new;
  p.offset = offset;
  p.pg = paging_of(cache);
  p.side_mask = 3;
  fill_signs(cache->seed, d, p.sign);
  copy_levels(cache->k, cache->k.thresholds, n_levels(cache->k) - 1, p.k_thr);
  copy_levels(cache->v, cache->v.thresholds, n_levels(cache->v) - 1, p.v_thr);
  const hipError_t e = tq::launch_quantize_append(p, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

size_t tq_decode_workspace_bytes(const tq_cache *cache, int q_heads, int length, int n_splits) {
  if (check_cache(cache) != TQ_OK) return 0;
  if (q_heads < cache->kv_heads || q_heads % cache->kv_heads) return 0;
  if (length < 0 || length > cache->capacity || n_splits < 0) return 0;
  tq::DecodeParams p;
  Variant v;
  return workspace_need(cache, q_heads, length, n_splits, &p, &v);
}

int tq_decode_attention(const tq_cache *cache, const void *q, int q_heads, int length, int n_splits,
                        float *out, float *scores, void *workspace, size_t workspace_bytes,
                        void *hip_stream) {
  return tq_decode_attention_sparse(cache, q, q_heads, length, n_splits, 0.0f, out, scores, workspace,
                                    workspace_bytes, hip_stream);
}

int tq_decode_attention_sparse(const tq_cache *cache, const void *q, int q_heads, int length, int n_splits,
                               float sparse_v, float *out, float *scores, void *workspace,
                               size_t workspace_bytes, void *hip_stream) {
  if (!(sparse_v >= 0.0f && sparse_v < 1.0f)) return TQ_ERR_ARG;
  int r = check_cache(cache);
  if (r != TQ_OK) return r;
  if (!q || !out) return TQ_ERR_ARG;
  if (q_heads < cache->kv_heads || q_heads % cache->kv_heads) return TQ_ERR_ARG;
  if (n_splits < 0) return TQ_ERR_ARG;
  if (length < 0 || length > cache->capacity) return TQ_ERR_CAPACITY;
  tq::DecodeParams p;
  Variant v;
  const size_t need = workspace_need(cache, q_heads, length, n_splits, &p, &v);
  if (need == 0) return TQ_ERR_ARG;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return TQ_ERR_WORKSPACE;
  p.q = static_cast<const uint16_t *>(q);
  p.out = out;
  p.scores = scores;
  p.ws = static_cast<float *>(workspace);
  p.counters = static_cast<unsigned *>(workspace);
  p.sparse_lg = sparse_v > 0.0f ? log2f(sparse_v) : -INFINITY;
  p.ws_part_off = tq::kCounterBytes;
  const hipError_t e = (v == kMfma) ? tq::launch_decode_mfma(p, static_cast<hipStream_t>(hip_stream))
                                    : tq::launch_decode_ref(p, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int tq_decode_attention_append(const tq_cache *cache, const void *k_new, const void *v_new, int offset,
                               const void *q, int q_heads, int length, int n_splits, float *out, float *scores,
                               void *workspace, size_t workspace_bytes, void *hip_stream) {
  // every argument of both steps is checked before anything is launched
  int r = check_cache(cache);
  if (r != TQ_OK) return r;
  if (!k_new || !v_new || !q || !out) return TQ_ERR_ARG;
  if (offset < 0 || offset >= cache->capacity) return TQ_ERR_CAPACITY;
  if (q_heads < cache->kv_heads || q_heads % cache->kv_heads) return TQ_ERR_ARG;
  if (n_splits < 0) return TQ_ERR_ARG;
  if (length < 0 || length > cache->capacity) return TQ_ERR_CAPACITY;
  tq::DecodeParams p;
  Variant v;
  const size_t need = workspace_need(cache, q_heads, length, n_splits, &p, &v);
  if (need == 0) return TQ_ERR_ARG;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return TQ_ERR_WORKSPACE;
  // one launch when the matrix-core kernel runs, no side is delegated, the
  // new position is attended and no scores are asked for; else the two
  // calls in order
  const auto plain = [](const tq_side &sd) {
    return sd.mode == TQ_SIDE_FP16 || sd.mode == TQ_SIDE_PACKED || sd.mode == TQ_SIDE_INT8;
  };
  if (v != kMfma || !plain(cache->k) || !plain(cache->v) || offset >= length || scores) {
    r = tq_quantize_append(cache, k_new, v_new, 1, offset, hip_stream);
    if (r != TQ_OK) return r;
    return tq_decode_attention_sparse(cache, q, q_heads, length, n_splits, 0.0f, out, scores, workspace,
                                      workspace_bytes, hip_stream);
  }
  p.q = static_cast<const uint16_t *>(q);
  p.out = out;
  p.scores = scores;
  p.ws = static_cast<float *>(workspace);
  p.counters = static_cast<unsigned *>(workspace);
  p.sparse_lg = -INFINITY;
  p.ws_part_off = tq::kCounterBytes;
  p.k_new = static_cast<const uint16_t *>(k_new);
  p.v_new = static_cast<const uint16_t *>(v_new);
  p.ap_offset = offset;
  p.ap_split = offset / p.cold_split_len;
  const float *kt = cache->k.mode == TQ_SIDE_PACKED ? cache->k.thresholds : nullptr;
  const float *vt = cache->v.mode == TQ_SIDE_PACKED ? cache->v.thresholds : nullptr;
  for (int i = 0; i < 16; ++i) {
    p.k_thr[i] = (kt && i < n_levels(cache->k) - 1) ? kt[i] : 0.0f;
    p.v_thr[i] = (vt && i < n_levels(cache->v) - 1) ? vt[i] : 0.0f;
  }
  const hipError_t e = tq::launch_decode_mfma(p, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int tq_decode_attention_noalloc(const tq_cache *cache, const void *q, int q_heads, int length, int n_splits,
                                float *out, float *scores, void *hip_stream) {
  int r = check_cache(cache);
  if (r != TQ_OK) return r;
  if (!q || !out) return TQ_ERR_ARG;
  if (q_heads < cache->kv_heads || q_heads % cache->kv_heads) return TQ_ERR_ARG;
  if (n_splits < 0) return TQ_ERR_ARG;
  if (length < 0 || length > cache->capacity) return TQ_ERR_CAPACITY;
  tq::DecodeParams p;
  Variant v;
  const size_t need = workspace_need(cache, q_heads, length, n_splits, &p, &v);
  if (need == 0) return TQ_ERR_ARG;
  if (need > tq::kScratchBytes) return TQ_ERR_SCRATCH;
  void *ws = nullptr;
  if (tq::scratch_workspace(static_cast<hipStream_t>(hip_stream), &ws) != hipSuccess) return TQ_ERR_HIP;
  return tq_decode_attention_sparse(cache, q, q_heads, length, n_splits, 0.0f, out, scores, ws, tq::kScratchBytes,
                                    hip_stream);
}

int tq_decode_workspace_init(void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (!workspace) return TQ_ERR_ARG;
  if (workspace_bytes < tq::kCounterBytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return TQ_ERR_WORKSPACE;
  const hipError_t e = tq::launch_zero_fill(workspace, tq::kCounterBytes, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int tq_dequantize(const tq_cache *cache, int side, int start, int count, float *out,
                  void *hip_stream) {
  int r = check_cache(cache);
  if (r != TQ_OK) return r;
  if (side != 0 && side != 1) return TQ_ERR_ARG;
  const tq_side &s = side ? cache->v : cache->k;
  if (s.mode == TQ_SIDE_FP16) return TQ_ERR_MODE;
  if (start < 0 || count < 0 || static_cast<long long>(start) + count > cache->capacity)
    return TQ_ERR_CAPACITY;
  if (count == 0) return TQ_OK;
  if (!out) return TQ_ERR_ARG;
  tq::DequantParams p;
  memset(&p, 0, sizeof(p));
  const int d = cache->head_dim;
  p.s = side_dev(s, d);
  p.out = out;
  p.batch = cache->batch;
  p.heads = cache->kv_heads;
  p.head_dim = d;
  p.capacity = cache->capacity;
  p.start = start;
  p.count = count;
  p.pg = paging_of(cache);
  fill_signs(cache->seed, d, p.sign);
  copy_levels(s, s.centroids, n_levels(s), p.cent);
  const hipError_t e = tq::launch_dequantize(p, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

int tq_read_probe(const void *buf, size_t bytes, unsigned *sink, void *hip_stream) {
  if (!sink || (bytes > 0 && !buf)) return TQ_ERR_ARG;
  if ((bytes & 15u) || (reinterpret_cast<uintptr_t>(buf) & 15u)) return TQ_ERR_ARG;
  const hipError_t e = tq::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // extern "C"
