/*
 * tq.h -- C ABI of libtq: TurboQuant KV-cache quantize-append and decode
 * attention computed from the packed cache, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (source pages: "TurboQuant KV Cache Quantization
 * in MLX-VLM", sections "The TurboQuantKVCache Class", "Quantization Codecs
 * and Bit Splitting", "How TurboQuant KV Cache Quantization Works" and the FAQ
 * on dequantization; "How to Use TurboQuant with the MLX-VLM CLI", section
 * "What Is TurboQuant?"; mlxcel "TurboQuant KV cache", sections "Available
 * modes" and "WHT head-dimension constraint"):
 *
 *   quantize   x (fp16, d values) -> n = ||x||_2 (fp32, one per token-head),
 *              y = H diag(s) x / (n sqrt(d)) with H the Sylvester Hadamard
 *              matrix and s a seeded sign vector, code_j = #{k : y_j > t_k}
 *              for the Lloyd-Max thresholds t of the coordinate pdf, packed
 *              LSB-first into uint32 words (code j at bits [b j, b j + b) of
 *              the row; word w holds bits [32 w, 32 w + 32)).
 *   dequantize x~ = n diag(s) H c[code] / sqrt(d).
 *   decode     out_h = softmax(q_h . K~^T / sqrt(d)) V~ for one query token
 *              per sequence, query head h reading KV head floor(h / G).
 *
 * Readings where the pages are silent: signs from SplitMix64 (sign j is
 * negative when the top bit of output j is set); one rotation per cache,
 * shared by K and V; ties go to the lower code; a zero row stores n = 0 and
 * codes L/2 - 1; no causal mask inside the attended length.
 *
 * Conventions for every entry point:
 *   - Status: 0 (TQ_OK) or a negative TQ_ERR_* code, returned synchronously.
 *     On any error nothing is launched and no caller memory is written.
 *   - Device pointers are caller-owned HIP device memory; the library never
 *     allocates, frees or synchronises.  Host pointers are read during the
 *     call only.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *     stream).  Results are visible after the caller synchronises the stream.
 *   - Layouts are dense, row-major, innermost index last.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  TQ_OK = 0,
  TQ_ERR_ARG = -1,       /* null pointer, negative size, bad q_heads, ...  */
  TQ_ERR_HEAD_DIM = -2,  /* head_dim not a power of two in [32, 256]
                            ("WHT head-dimension constraint": no padding)   */
  TQ_ERR_BITS = -3,      /* packed side with bits outside [1, 8]            */
  TQ_ERR_CAPACITY = -4,  /* rows outside [0, capacity)                      */
  TQ_ERR_WORKSPACE = -5, /* workspace missing or smaller than required      */
  TQ_ERR_MODE = -6,      /* unsupported side mode or mode combination       */
  TQ_ERR_HIP = -7,       /* the HIP runtime reported a launch error         */
  TQ_ERR_SCRATCH = -8    /* tq_decode_attention_noalloc: the call needs more
                            than TQ_NOALLOC_SCRATCH_BYTES of workspace      */
};

/* How one side (K or V) of a cache is stored ("Available modes": fp16 K with
 * TurboQuant V, TurboQuant K and V, and the delegated hot/cold V split). */
enum {
  TQ_SIDE_FP16 = 0,      /* plain fp16 rows                                 */
  TQ_SIDE_PACKED = 1,    /* TurboQuant codes + fp32 norms                   */
  TQ_SIDE_DELEGATED = 2, /* V only: newest `hot` tokens fp16 in a ring
                            (slot = position mod hot), older tokens packed  */
  TQ_SIDE_INT8 = 3       /* per-token INT8 absmax (mlxcel "TurboQuant KV cache",
                            "Available modes"): codes int8 [B][Hkv][capacity][d]
                            in `codes` (d / 4 words a row, coordinate j in byte
                            j), the per-row scale max|x| / 127 in `norms`; no
                            rotation, codebook or bit width (bits ignored)     */
};

#define TQ_MIN_BITS 1
#define TQ_MAX_BITS 8
#define TQ_MIN_HEAD_DIM 32
#define TQ_MAX_HEAD_DIM 256

/* Bit split of a (possibly fractional) budget: keys get floor(bits), values
 * ceil(bits) ("Quantization Codecs and Bit Splitting").  Returns TQ_ERR_BITS
 * unless 1 <= floor(bits) and ceil(bits) <= 8; TQ_ERR_ARG on null outputs. */
int tq_split_bits(double bits, int *k_bits, int *v_bits);

/* uint32 words per packed row: ceil(bits * head_dim / 32).  Returns the count
 * (> 0), or TQ_ERR_HEAD_DIM / TQ_ERR_BITS. */
int tq_row_words(int head_dim, int bits);

/* Sign vector of the rotation for `seed`: bit j of sign_words[j / 32] is set
 * when s_j = -1.  sign_words must hold head_dim / 32 words (host memory).
 * ("How TurboQuant KV Cache Quantization Works": random Hadamard transform;
 * SplitMix64 of Steele, Lea and Flood (2014) is the sign source.) */
int tq_sign_words(uint64_t seed, int head_dim, uint32_t *sign_words);

/* Lloyd-Max codebook for one coordinate of a uniform unit vector in
 * R^head_dim, whose density is proportional to (1 - x^2)^((head_dim - 3)/2)
 * (the "Beta-PDF Lloyd-Max quantizer").  Host only, deterministic, double
 * precision; takes milliseconds for bits <= 5 and up to seconds for 8 bits,
 * so build once per (head_dim, bits) and keep the result.
 *   centroids:  [1 << bits], ascending, antisymmetric (c_k = -c_{L-1-k}).
 *   thresholds: [(1 << bits) - 1], midpoints of neighbouring centroids; the
 *               middle one is exactly 0.
 * head_dim must be a power of two in [2, 65536] here (the quantizer itself
 * only accepts [32, 256]). */
int tq_build_codebook(int head_dim, int bits, double *centroids,
                      double *thresholds);

/* One side of one layer's cache.  All buffers are caller-owned. */
typedef struct tq_side {
  int mode;                /* TQ_SIDE_*                                       */
  int bits;                /* PACKED / DELEGATED: code width in [1, 8]        */
  const float *centroids;  /* HOST fp32 [1 << bits]: the side's codebook,
                              normally tq_build_codebook rounded to fp32      */
  const float *thresholds; /* HOST fp32 [(1 << bits) - 1]                     */
  uint32_t *codes;         /* DEVICE [B][Hkv][capacity][row_words]           */
  float *norms;            /* DEVICE [B][Hkv][capacity]                      */
  uint16_t *fp16;          /* DEVICE fp16 bits: FP16 -> [B][Hkv][capacity][d];
                              DELEGATED -> hot ring [B][Hkv][hot][d]          */
  int hot;                 /* DELEGATED: ring length (>= 1)                   */
} tq_side;

/* One layer's cache.  K may be FP16, PACKED or INT8; V may be FP16, PACKED,
 * DELEGATED or INT8.  `seed` selects the rotation shared by both sides.
 *
 * Paged storage (mlxcel "TurboQuant KV cache", "Paged cache and server
 * batching": TurboQuant modes in a block-table decode layout).  With
 * block_table NULL (zero-initialised descriptor) every side is contiguous as
 * described in tq_side.  With a block table, the codes, norms and fp16 rows
 * of both sides live in pools of fixed-size blocks instead:
 *   codes [num_blocks][Hkv][block_size][row_words], norms
 *   [num_blocks][Hkv][block_size], fp16 rows [num_blocks][Hkv][block_size][d],
 * and position t of sequence b sits in block block_table[b][t / block_size]
 * at row t % block_size.  The DELEGATED hot ring stays [B][Hkv][hot][d].
 *   block_table: DEVICE int32 [B][max_blocks]; entries are block indices of
 *                the pools.  The library does not read device memory on the
 *                host, so entries are checked on the device: an entry
 *                outside [0, num_blocks) makes its positions read as zero
 *                rows (score 0, value 0; they still count in the softmax)
 *                and an append to them writes nothing, so a bad entry never
 *                reaches memory outside the pools.  Blocks may be shared
 *                between sequences for positions they share; an append must
 *                not write different rows into a shared block (copy it
 *                first).
 *   block_size:  positions per block, a multiple of 32.
 *   max_blocks:  table row length; capacity must equal max_blocks * block_size.
 *   num_blocks:  blocks in each pool (>= 1).
 * Errors: TQ_ERR_ARG if block_size, max_blocks or num_blocks is invalid or
 * capacity does not match. */
typedef struct tq_cache {
  int batch;
  int kv_heads;
  int head_dim;
  int capacity;  /* positions per (batch, kv head) */
  uint64_t seed;
  tq_side k;
  tq_side v;
  const int32_t *block_table; /* NULL: contiguous sides */
  int block_size;
  int max_blocks;
  int num_blocks;
} tq_cache;

/* Quantize-append ("update_and_fetch" of the TurboQuantKVCache; one launch
 * handles K and V, as the fused quantize path does).
 * k_new, v_new: DEVICE fp16 [B][Hkv][n_new][d].  Writes positions
 * [offset, offset + n_new) of each side and nothing else:
 *   PACKED    -> codes/norms rows at those positions;
 *   FP16      -> fp16 rows at those positions;
 *   DELEGATED -> for each new position p, the ring slot p mod hot is first
 *                evicted (its previous occupant, position p - hot, is
 *                quantized into the packed cold rows) and then overwritten;
 *                new positions that are already older than the newest `hot`
 *                go straight to the cold rows.  Positions must be appended
 *                in order (offset = current length) for the ring to hold the
 *                newest tokens;
 *   INT8      -> per row, scale = fp32(max|x| / 127) in `norms` and code_j =
 *                round(127 x_j / max|x|) (to nearest, ties to even; the exact
 *                value, not a float32 approximation of it) in `codes`; a zero
 *                row stores scale 0 and codes 0.
 * Errors: TQ_ERR_CAPACITY if offset < 0 or offset + n_new > capacity.
 * n_new = 0 is a no-op returning TQ_OK. */
int tq_quantize_append(const tq_cache *cache, const void *k_new,
                       const void *v_new, int n_new, int offset,
                       void *hip_stream);

/* Bytes of workspace tq_decode_attention needs for this shape (0 on invalid
 * arguments).  n_splits = 0 picks the library's split of the context.  The
 * size is at least TQ_WORKSPACE_COUNTER_BYTES. */
size_t tq_decode_workspace_bytes(const tq_cache *cache, int q_heads,
                                 int length, int n_splits);

/* The decode workspace starts with TQ_WORKSPACE_COUNTER_BYTES of per-unit
 * arrival counters (the last block of a (batch, KV head) unit to finish
 * merges the context splits).  They must read zero before the workspace's
 * first decode; every successful decode leaves them zero again, so one
 * set-up serves every later call, whatever its shape.  A workspace whose
 * counters are not zero gives undefined output (a merge may run early or
 * not at all).  Zero them with tq_decode_workspace_init or any zero fill. */
#define TQ_WORKSPACE_COUNTER_BYTES (256u * 1024u)

/* Zero the counter region of a decode workspace on `hip_stream` (a store
 * kernel, no memset, so it may be recorded into a HIP graph).
 *   workspace: DEVICE, 256-byte aligned, workspace_bytes >=
 *              TQ_WORKSPACE_COUNTER_BYTES (else TQ_ERR_WORKSPACE).
 * Errors: TQ_ERR_ARG on a null workspace. */
int tq_decode_workspace_init(void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/* Decode attention over positions [0, length) straight from the packed cache
 * ("How TurboQuant KV Cache Quantization Works": scores from the compressed
 * representation).  Packed K is scored as n_i <R q, c[code_i]>; packed V is
 * accumulated in the rotated domain and rotated back once per output head.
 * INT8 rows are used as scale_i code_i, in the original domain.
 * A DELEGATED V is attended as "the newest `hot` positions from the ring,
 * older ones packed", with newest meaning the last `length` positions: the
 * ring holds the newest `hot` positions appended, so length must equal the
 * number of positions appended (a shorter length reads ring slots that later
 * appends have overwritten).
 *   q:      DEVICE fp16 [B][q_heads][d]; q_heads a multiple of kv_heads.
 *   out:    DEVICE fp32 [B][q_heads][d].
 *   scores: DEVICE fp32 [B][q_heads][length] or NULL; when given, receives
 *           the scaled logits q . k~ / sqrt(d).
 *   workspace: DEVICE, >= tq_decode_workspace_bytes(...), 256-byte aligned,
 *           its counters zero before its first use (see
 *           TQ_WORKSPACE_COUNTER_BYTES).  It holds per-split partial
 *           results; calls that share a workspace must not overlap.
 *   n_splits: 0 = automatic, else the number of context splits asked
 *           for (>= 1): pieces of equal length.  The matrix-core kernel
 *           rounds each piece up to a multiple of 32 positions (what it
 *           reads as one chunk), so it may use fewer splits than asked,
 *           never more.
 * length = 0 writes zeros to out. */
int tq_decode_attention(const tq_cache *cache, const void *q, int q_heads,
                        int length, int n_splits, float *out, float *scores,
                        void *workspace, size_t workspace_bytes,
                        void *hip_stream);

/* Sparse-V decode (mlxcel "TurboQuant KV cache", "CLI and server flags":
 * the sparse-V threshold, 0 disabling it): tq_decode_attention, except that
 * the value contribution of positions whose softmax weight is below
 * `sparse_v` times the largest weight may be dropped.  The softmax
 * denominator keeps every position; only values are skipped, and only where
 * a whole group of positions (a 32-position chunk of the matrix-core kernel,
 * one position in the plain kernel) is below the threshold, judged against
 * a running maximum that never exceeds the final one.  So each dropped
 * position i has p_i < sparse_v (p relative to the largest weight), and
 * every output element moves by at most sum over such i of p_i |v_i| / sum p.
 * In the matrix-core kernel that maximum also includes what the block's
 * other waves saw in their first chunks (exchanged at one barrier), so
 * which groups are dropped depends only on the data: results are
 * bit-reproducible, as are the exact decode's.
 *   sparse_v: in [0, 1); 0 is exactly tq_decode_attention.
 * Errors: as tq_decode_attention; TQ_ERR_ARG if sparse_v is outside [0, 1). */
int tq_decode_attention_sparse(const tq_cache *cache, const void *q, int q_heads,
                               int length, int n_splits, float sparse_v, float *out,
                               float *scores, void *workspace, size_t workspace_bytes,
                               void *hip_stream);

/* One decode step's append-then-attend in one call ("TurboQuant KV Cache
 * Quantization in MLX-VLM", "Manual Cache Operations": quantize the new K/V
 * into the cache, then score from the compressed cache): the same results
 * as tq_quantize_append(cache, k_new, v_new, 1, offset, stream) followed by
 * tq_decode_attention(cache, q, q_heads, length, n_splits, out, scores,
 * workspace, workspace_bytes, stream).
 *   k_new, v_new: device fp16 [B][Hkv][1][d], the new position of every
 *                 sequence; written at row `offset` (0 <= offset < capacity).
 *   the rest: as tq_decode_attention (the same workspace size).
 * Where the matrix-core decode takes the shape, no side is delegated,
 * offset < length and `scores` is NULL, this is one launch: in the
 * split that holds `offset`, the wave that reads the position's chunk
 * encodes and writes the new rows first, so the step pays no separate
 * launch.  Otherwise (delegated V, other shapes, offset >= length, scores
 * requested) it makes the two calls in order on `hip_stream`.  The rows written are those tq_quantize_append defines, up
 * to rounding: the one-launch path sums the norm and the rotation of packed
 * rows in another order, so a norm may differ in its last bits and a
 * coordinate within rounding of a threshold may take the neighbouring code
 * (fp16 and INT8 rows are the same).
 * Errors: as tq_quantize_append (with n_new = 1) and tq_decode_attention,
 * all checked before anything is launched. */
int tq_decode_attention_append(const tq_cache *cache, const void *k_new, const void *v_new,
                               int offset, const void *q, int q_heads, int length, int n_splits,
                               float *out, float *scores, void *workspace, size_t workspace_bytes,
                               void *hip_stream);

/* tq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a fixed static device
 * array of TQ_NOALLOC_SCRATCH_BYTES per GPU, which the library holds until
 * the process ends; nothing is allocated or freed.  The first call on a
 * device looks the array up and clears its counters on `hip_stream`.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, threads) race and must be serialised by the caller.
 * Results are those of tq_decode_attention (the same kernels and splits).
 * Errors: as tq_decode_attention; TQ_ERR_SCRATCH (nothing launched) when
 * tq_decode_workspace_bytes for the call exceeds TQ_NOALLOC_SCRATCH_BYTES. */
#define TQ_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int tq_decode_attention_noalloc(const tq_cache *cache, const void *q,
                                int q_heads, int length, int n_splits,
                                float *out, float *scores, void *hip_stream);

/* Dequantize packed rows [start, start + count) of one side (0 = K, 1 = V;
 * for a DELEGATED V this reads the packed cold rows) into DEVICE fp32
 * out[B][Hkv][count][d] (the FAQ's "dequantize" back to float32).  A check
 * path; FP16 sides return TQ_ERR_MODE. */
int tq_dequantize(const tq_cache *cache, int side, int start, int count,
                  float *out, void *hip_stream);

/* Static description of a status code. */
const char *tq_status_string(int status);

/* Measurement aid, not part of the method: stream-read `bytes` of DEVICE
 * memory at `buf` (16-byte loads, a few in flight per thread, one block per
 * compute unit) and write the xor of all its 32-bit words to DEVICE *sink.
 * Timing it gives the HBM read bandwidth a plain streaming kernel attains
 * on this GPU, against which the decode's bandwidth can be read (the
 * published peak stays the roofline).  `bytes` must be a multiple of 16 and
 * `buf` 16-byte aligned, else TQ_ERR_ARG; 0 bytes writes 0 to *sink. */
int tq_read_probe(const void *buf, size_t bytes, unsigned *sink,
                  void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
