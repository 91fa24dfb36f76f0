// Decode attention straight from the packed cache: the plain split-context
// variant ("TurboQuant KV Cache Quantization in MLX-VLM", "How TurboQuant KV
// Cache Quantization Works": scores from the compressed representation; FAQ
// on dequantization: the stored rotation and codebooks).  It serves every
// cache layout the matrix-core kernel does not: head_dim other than 128,
// INT8 sides, code widths other than 3 or 4 bits for K and 4 for V, more
// than eight query heads per KV head.
//
// Grid (n_splits, B * Hkv, head groups); one block handles up to eight query
// heads of one KV head over one contiguous range of positions:
//   1. q is rotated once: R q = H diag(s) q / sqrt(d) by butterflies in LDS;
//      the softmax scale 1/sqrt(d) and log2(e) are folded in.
//   2. the range is walked in tiles of 64 positions (32 where a tile's
//      rows do not fit the lanes' prefetch slots).  Each tile's K and V
//      rows (packed codes, INT8 codes or fp16, as stored) are copied to LDS
//      with row-contiguous loads, 16 bytes a lane where rows allow it; the
//      next tile's loads are in flight while the current one is computed.
//   3. scores from the LDS rows: n_i <R q, c[code_i]> (packed K), s_i q .
//      code_i (INT8 K) or q . k_i (fp16 K).  A lane takes one position and
//      a slice of the coordinates for every head of the block; the slices'
//      partial sums are added in the softmax step.
//   4. online softmax per head (base-2 exponent): the running maximum and
//      sum, and the factor that rescales the accumulators.
//   5. value accumulation: a lane owns one coordinate j for every head and
//      takes every (256 / d)-th position of the tile.  Packed rows add
//      p_i n_i c[code_i,j] in the rotated domain; fp16 rows (fp16 V, the
//      delegated hot window) add p_i v_ij and INT8 rows p_i s_i code_ij in
//      the original domain.  The lane groups' sums are added at the end.
//   6. partial (max, sum, rotated sum, plain sum) to the workspace.
// A second kernel merges the splits by their maxima, applies the inverse
// rotation diag(s) H / sqrt(d) once per output head, adds the plain part and
// divides by the sum.
#include <math.h>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxGroupHeads = 8;   // query heads per block

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// LDS plan of one block (offsets in 32-bit words).  Row strides are odd so
// that the same word of consecutive rows falls in different banks.  HB is
// the head count the block's arrays are sized for (1, 2, 4 or 8, at least
// its gb heads); unused heads carry zero weights.
struct RefLayout {
  int gb, ngroups, hb;      // query heads per block, blocks per KV head, array heads
  int kw, vw_cold, vw_hot;  // words of a staged K row, packed / INT8 V row, fp16 V row
  int sk, sv;               // LDS row strides
  int qr, sp, pw, kt, vt, kn, vn, ck, cv, al, total;
};

// tt: positions per tile (32 or 64).
__host__ __device__ inline RefLayout ref_layout(const DecodeParams &p, int D, int tt) {
  RefLayout L;
  const int G = p.q_heads / p.kv_heads;
  L.ngroups = (G + kMaxGroupHeads - 1) / kMaxGroupHeads;
  L.gb = (G + L.ngroups - 1) / L.ngroups;
  L.hb = L.gb <= 1 ? 1 : (L.gb <= 2 ? 2 : (L.gb <= 4 ? 4 : 8));
  L.kw = p.k.mode == TQ_SIDE_FP16 ? D / 2 : p.k.words;
  L.vw_cold = p.v.mode == TQ_SIDE_FP16 ? D / 2 : p.v.words;
  L.vw_hot = (p.v.mode == TQ_SIDE_FP16 || p.v.mode == TQ_SIDE_DELEGATED) ? D / 2 : L.vw_cold;
  L.sk = L.kw | 1;
  L.sv = (L.vw_cold > L.vw_hot ? L.vw_cold : L.vw_hot) | 1;
  int o = 0;
  L.qr = o; o += L.hb * D;                 // rotated, scaled queries [head][d]
  L.sp = o; o += kBlock * L.hb;            // partial scores [part][head][pos] (256 / tt x tt x hb);
                                           // at the end the value sums [lane group][head][d]
                                           // (256 / d x hb x d)
  L.pw = o; o += tt * L.hb;                // weight times the V row's norm or scale [pos][head]
  L.kt = o; o += tt * L.sk;                // K tile
  L.vt = o; o += tt * L.sv;                // V tile
  L.kn = o; o += tt;                       // K norms / scales (1 for fp16 rows)
  L.vn = o; o += tt;                       // V norms / scales (1 for fp16 rows)
  L.ck = o; o += kMaxLevels;               // centroids
  L.cv = o; o += kMaxLevels;
  L.al = o; o += kMaxGroupHeads;           // per-head rescale factor of the tile
  L.total = o;
  return L;
}

// First position served from fp16 storage: all of an fp16 V, the hot window
// of a delegated V, none otherwise.
__device__ __forceinline__ int v_hot_start(const DecodeParams &p) {
  if (p.v.mode == TQ_SIDE_FP16) return 0;
  if (p.v.mode == TQ_SIDE_DELEGATED) return p.length - p.v.hot;
  return 0x7fffffff;
}

// fp16 row r of a side, or the zero row where r < 0 (a block outside the pools)
template <int D>
__device__ __forceinline__ const uint32_t *fp16_row_or_zero(const uint16_t *base, long r) {
  return r < 0 ? kZeroRow : reinterpret_cast<const uint32_t *>(base + r * D);
}

// Start of piece `piece` (GW words) of the stored row of position t, or null
// where that row kind is shorter (the cold rows of a delegated V).  A
// position in a block outside the paged pools reads the zero row where the
// row is fp16; a code row (packed or INT8) is read from the pool's row 0
// instead, and its norm (scale) reads 0 (Stager::load), so the row still
// contributes exactly nothing.  (This shape keeps the kernel at the register
// count of the unguarded one.)
template <int D, int GW>
__device__ __forceinline__ const uint32_t *piece_src(const DecodeParams &p, const RefLayout &L, long bk, int t,
                                                     bool is_k, int piece, int hot_start) {
  const uint32_t *src;
  if (is_k) {
    src = p.k.mode == TQ_SIDE_FP16 ? fp16_row_or_zero<D>(p.k.fp16, cache_row(p.pg, bk, t, p.capacity))
                                   : p.k.codes + max(cache_row(p.pg, bk, t, p.capacity), 0L) * p.k.words;
  } else if (t >= hot_start) {
    if (piece * GW >= L.vw_hot) return nullptr;
    src = p.v.mode == TQ_SIDE_FP16
              ? fp16_row_or_zero<D>(p.v.fp16, cache_row(p.pg, bk, t, p.capacity))
              : reinterpret_cast<const uint32_t *>(p.v.fp16 + (bk * p.v.hot + t % p.v.hot) * D);
  } else {
    if (piece * GW >= L.vw_cold) return nullptr;
    src = p.v.codes + max(cache_row(p.pg, bk, t, p.capacity), 0L) * p.v.words;
  }
  return src + piece * GW;
}

// Copy of one tile's K and V rows from HBM to LDS.  The tile is cut into
// GW-word pieces, K rows first; lane l owns pieces l + 256 u.  For the first
// four (u < 4: every piece of a 32-position tile at head_dim <= 128 with
// 16-byte loads, and of the 64-position tiles the host picks) the row, the
// piece and the LDS offset are the same for every tile, so they are worked
// out once, and the loads of the next tile are issued before the current
// one is scored and stored after it, so HBM latency overlaps compute.
// Pieces beyond those (fp16 rows at head_dim 256, 4-byte loads) are copied
// when the tile is stored.
template <int D, int GW, int TT>
struct Stager {
  static constexpr int kSlots = 4;
  u32x4_t buf[kSlots];
  int row[kSlots];      // tile row of the piece, -1 = no piece
  int piece[kSlots];    // piece index within the row
  int dst[kSlots];      // LDS word offset
  bool is_k[kSlots];
  bool live[kSlots];    // the piece was loaded for the current tile
  float norm;           // lanes 0..TT-1: K norm, 64..63+TT: V norm of the tile row
  int norm_dst;         // LDS word offset of that norm, -1 = none
  int kg, vg;           // pieces per K row, per V row (the longer kind)
  int tb, nt;           // the loaded tile

  __device__ void init(const RefLayout &L) {
    const int tid = threadIdx.x;
    kg = L.kw / GW;
    const int vgc = L.vw_cold / GW, vgh = L.vw_hot / GW;
    vg = vgc > vgh ? vgc : vgh;
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int i = tid + u * kBlock;
      row[u] = -1;
      if (i < TT * (kg + vg)) {
        is_k[u] = i < TT * kg;
        const int ii = is_k[u] ? i : i - TT * kg;
        const int per = is_k[u] ? kg : vg;
        row[u] = ii / per;
        piece[u] = ii - row[u] * per;
        dst[u] = (is_k[u] ? L.kt + row[u] * L.sk : L.vt + row[u] * L.sv) + piece[u] * GW;
      }
    }
    norm_dst = tid < TT ? L.kn + tid : ((tid >= 64 && tid < 64 + TT) ? L.vn + tid - 64 : -1);
  }

  // Issue the loads of positions [t, t + n).
  __device__ void load(const DecodeParams &p, const RefLayout &L, long bk, int t, int n, int hot_start) {
    const int tid = threadIdx.x;
    tb = t;
    nt = n;
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      live[u] = false;
      if (row[u] >= 0 && row[u] < n) {
        const uint32_t *src = piece_src<D, GW>(p, L, bk, t + row[u], is_k[u], piece[u], hot_start);
        if (src) {
          if (GW == 4) {
            buf[u] = *reinterpret_cast<const u32x4_t *>(src);
          } else {
            buf[u].x = *src;
          }
          live[u] = true;
        }
      }
    }
    norm = 1.0f;
    if (tid < n) {
      if (p.k.mode != TQ_SIDE_FP16) {
        const long r = cache_row(p.pg, bk, t + tid, p.capacity);
        norm = r < 0 ? 0.0f : p.k.norms[r];
      }
    } else if (tid >= 64 && tid < 64 + n && t + tid - 64 < hot_start) {
      const long r = cache_row(p.pg, bk, t + tid - 64, p.capacity);
      norm = r < 0 ? 0.0f : p.v.norms[r];
    }
  }

  // Write the loaded tile to LDS (waits for its loads), and copy the pieces
  // beyond the lanes' slots.
  __device__ void store(const DecodeParams &p, const RefLayout &L, long bk, int hot_start, uint32_t *lds) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      if (live[u]) {
        lds[dst[u]] = buf[u].x;
        if (GW == 4) {
          lds[dst[u] + 1] = buf[u].y;
          lds[dst[u] + 2] = buf[u].z;
          lds[dst[u] + 3] = buf[u].w;
        }
      }
    }
    if (norm_dst >= 0) reinterpret_cast<float *>(lds)[norm_dst] = norm;
    for (int i = threadIdx.x + kSlots * kBlock; i < TT * (kg + vg); i += kBlock) {
      const bool k = i < TT * kg;
      const int ii = k ? i : i - TT * kg;
      const int per = k ? kg : vg;
      const int r = ii / per, pc = ii - r * per;
      if (r >= nt) continue;
      const uint32_t *src = piece_src<D, GW>(p, L, bk, tb + r, k, pc, hot_start);
      if (!src) continue;
      const int o = (k ? L.kt + r * L.sk : L.vt + r * L.sv) + pc * GW;
#pragma unroll
      for (int e = 0; e < GW; ++e) lds[o + e] = src[e];
    }
  }
};

// fp16 element j of a row held as 32-bit words.
__device__ __forceinline__ float half_at(const uint32_t *row, int j) {
  return h2f(static_cast<uint16_t>(row[j >> 1] >> (16 * (j & 1))));
}

// Value sums of one run of positions (every TS-th from `first` below
// `end`) for one coordinate j and all HB heads: acc[h] += w[pos][h] * value.
// KIND 0: packed rows (centroid of the code), 1: INT8 rows (the code), 2:
// fp16 rows.
template <int D, int HB, int KIND>
__device__ __forceinline__ void accumulate(float (&acc)[HB], const uint32_t *vt, int sv, const float *pw,
                                           const float *cv, int bits, int j, int first, int end) {
  constexpr int TS = kBlock / D;
#pragma unroll 4
  for (int tok = first; tok < end; tok += TS) {
    const uint32_t *row = vt + tok * sv;
    float x;
    if (KIND == 0) {
      x = cv[extract_code(row, bits, j)];
    } else if (KIND == 1) {
      x = int8_at(row[j >> 2], j);
    } else {
      x = half_at(row, j);
    }
    const float *w = pw + tok * HB;
#pragma unroll
    for (int h = 0; h < HB; ++h) acc[h] += w[h] * x;
  }
}

// GW: words per staging load (4 = 16-byte loads; the host picks 4 when every
// row kind is a multiple of 16 bytes and the storage is 16-byte aligned).
// HB: heads the per-lane arrays hold (>= the block's heads).  TT: positions
// per tile, 64 where a tile's pieces fit the lanes' prefetch slots, else 32.
template <int D, int GW, int HB, int TT>
__global__ __launch_bounds__(kBlock) void decode_split_kernel(const DecodeParams p) {
  extern __shared__ __align__(16) uint32_t lds[];
  const RefLayout L = ref_layout(p, D, TT);
  float *qr = reinterpret_cast<float *>(lds + L.qr);
  float *sp = reinterpret_cast<float *>(lds + L.sp);
  float *pw = reinterpret_cast<float *>(lds + L.pw);
  const uint32_t *kt = lds + L.kt;
  const uint32_t *vt = lds + L.vt;
  const float *kn = reinterpret_cast<const float *>(lds + L.kn);
  const float *vn = reinterpret_cast<const float *>(lds + L.vn);
  float *ck = reinterpret_cast<float *>(lds + L.ck);
  float *cv = reinterpret_cast<float *>(lds + L.cv);
  float *al = reinterpret_cast<float *>(lds + L.al);

  const int tid = threadIdx.x;
  const int G = p.q_heads / p.kv_heads;
  const int split = blockIdx.x;
  const long bk = blockIdx.y;
  const int g0 = blockIdx.z * L.gb;
  const int gn = min(L.gb, G - g0);  // query heads of this block, 1 <= gn <= HB
  const int b = static_cast<int>(bk / p.kv_heads), kv = static_cast<int>(bk % p.kv_heads);
  const int t0 = split * p.split_len;
  const int t1 = min(p.length, t0 + p.split_len);
  const long hq0 = static_cast<long>(b) * p.q_heads + static_cast<long>(kv) * G + g0;
  const int hot_start = v_hot_start(p);

  for (int i = tid; i < kMaxLevels; i += kBlock) {
    ck[i] = p.k_cent[i];
    cv[i] = p.v_cent[i];
  }
  const bool k_packed = p.k.mode == TQ_SIDE_PACKED;
  for (int i = tid; i < HB * D; i += kBlock) {
    const float x = i < gn * D ? h2f(p.q[hq0 * D + i]) : 0.0f;
    qr[i] = k_packed ? x * sign_of(p.sign, i % D) : x;
  }
  __syncthreads();
  if (k_packed) {
    for (int s = 1; s < D; s <<= 1) {
      for (int i = tid; i < gn * D / 2; i += kBlock) {
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
  for (int i = tid; i < gn * D; i += kBlock) qr[i] *= qscale;

  // score lanes: position stok, coordinates [part, part + 1) * D / kParts
  constexpr int kParts = kBlock / TT;
  const int stok = tid % TT, part = tid / TT;
  constexpr int kCpl = D / kParts;
  // softmax lanes: in pass ps, the TT lanes of group `part` handle head
  // part + ps * kParts, lane stok position stok
  constexpr int kPasses = (HB * TT + kBlock - 1) / kBlock;
  float m_run[kPasses], l_run[kPasses];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    m_run[ps] = -INFINITY;
    l_run[ps] = 0.0f;
  }
  // value lanes: coordinate vj, every TS-th position from vsub
  constexpr int TS = kBlock / D;
  const int vj = tid % D, vsub = tid / D;
  float acc_rot[HB], acc_plain[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) acc_rot[h] = acc_plain[h] = 0.0f;

  Stager<D, GW, TT> st;
  st.init(L);
  __syncthreads();
  if (t0 < t1) st.load(p, L, bk, t0, min(TT, t1 - t0), hot_start);
  for (int tb = t0; tb < t1; tb += TT) {
    const int nt = min(TT, t1 - tb);
    st.store(p, L, bk, hot_start, lds);
    __syncthreads();
    if (tb + TT < t1) st.load(p, L, bk, tb + TT, min(TT, t1 - tb - TT), hot_start);

    // scores: partial dot products of one position over a slice of the
    // coordinates, for every head
    {
      float acc[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) acc[h] = 0.0f;
      if (stok < nt) {
        const uint32_t *row = kt + stok * L.sk;
        const int j0 = part * kCpl;
        if (k_packed) {
#pragma unroll 4
          for (int j = j0; j < j0 + kCpl; ++j) {
            const float c = ck[extract_code(row, p.k.bits, j)];
#pragma unroll
            for (int h = 0; h < HB; ++h) acc[h] += qr[h * D + j] * c;
          }
        } else if (p.k.mode == TQ_SIDE_INT8) {
#pragma unroll
          for (int j = j0; j < j0 + kCpl; j += 4) {
            const uint32_t w = row[j >> 2];
            const float x0 = int8_at(w, 0), x1 = int8_at(w, 1), x2 = int8_at(w, 2), x3 = int8_at(w, 3);
#pragma unroll
            for (int h = 0; h < HB; ++h) {
              const float4 q4 = *reinterpret_cast<const float4 *>(qr + h * D + j);
              acc[h] += q4.x * x0 + q4.y * x1 + q4.z * x2 + q4.w * x3;
            }
          }
        } else {
#pragma unroll
          for (int j = j0; j < j0 + kCpl; j += 2) {
            const float x0 = half_at(row, j), x1 = half_at(row, j + 1);
#pragma unroll
            for (int h = 0; h < HB; ++h) {
              const float2 q2 = *reinterpret_cast<const float2 *>(qr + h * D + j);
              acc[h] += q2.x * x0 + q2.y * x1;
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < HB; ++h) sp[(part * HB + h) * TT + stok] = acc[h];
    }
    __syncthreads();

    // online softmax, TT lanes per head
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int sh = part + ps * kParts;
      if (sh < HB) {
        if (sh < gn) {
          float s = -INFINITY;
          if (stok < nt) {
            float a = 0.0f;
#pragma unroll
            for (int q = 0; q < kParts; ++q) a += sp[(q * HB + sh) * TT + stok];
            s = a * kn[stok];
            if (p.scores) p.scores[(hq0 + sh) * p.length + tb + stok] = s * kLn2;
          }
          const float m_new = fmaxf(m_run[ps], group_max<TT>(s));
          const float alpha = (m_run[ps] == -INFINITY) ? 0.0f : exp2f(m_run[ps] - m_new);
          float w = (stok < nt && m_new != -INFINITY) ? exp2f(s - m_new) : 0.0f;
          l_run[ps] = l_run[ps] * alpha + group_sum<TT>(w);
          m_run[ps] = m_new;
          // sparse-V: drop the value of a position whose weight, relative to
          // the running maximum, is below the threshold (it stays in the sum)
          if (p.sparse_lg != -INFINITY && !(s - m_new >= p.sparse_lg)) w = 0.0f;
          pw[stok * HB + sh] = stok < nt ? w * vn[stok] : 0.0f;
          if (stok == 0) al[sh] = alpha;
        } else {
          pw[stok * HB + sh] = 0.0f;
          if (stok == 0) al[sh] = 0.0f;
        }
      }
    }
    __syncthreads();

    // values: coordinate vj of every head over this lane's positions; the
    // cold (packed or INT8) positions first, then the fp16 ones
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      acc_rot[h] *= al[h];
      acc_plain[h] *= al[h];
    }
    const int nc = min(nt, max(0, hot_start - tb));
    if (nc > 0) {
      if (p.v.mode == TQ_SIDE_INT8) {
        accumulate<D, HB, 1>(acc_plain, vt, L.sv, pw, cv, p.v.bits, vj, vsub, nc);
      } else {
        accumulate<D, HB, 0>(acc_rot, vt, L.sv, pw, cv, p.v.bits, vj, vsub, nc);
      }
    }
    if (nc < nt) accumulate<D, HB, 2>(acc_plain, vt, L.sv, pw, cv, p.v.bits, vj, nc + vsub, nt);
    __syncthreads();
  }

  const DecodeWorkspace lay = decode_workspace_layout(p.batch, p.q_heads, p.n_splits, D);
  float *ml = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + lay.ml_off);
  float *orot = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + lay.orot_off);
  float *ohot = reinterpret_cast<float *>(reinterpret_cast<char *>(p.ws) + lay.ohot_off);
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int sh = part + ps * kParts;
    if (sh < gn && stok == 0) {
      ml[((hq0 + sh) * p.n_splits + split) * 2 + 0] = m_run[ps];
      ml[((hq0 + sh) * p.n_splits + split) * 2 + 1] = l_run[ps];
    }
  }
  // sum the TS lane groups' value sums (through LDS), then write them
  float *red = sp;  // [TS][HB][D]
  for (int pass = 0; pass < 2; ++pass) {
    float *dst = pass == 0 ? orot : ohot;
#pragma unroll
    for (int h = 0; h < HB; ++h) red[(vsub * HB + h) * D + vj] = pass == 0 ? acc_rot[h] : acc_plain[h];
    __syncthreads();
    for (int o = tid; o < gn * D; o += kBlock) {
      const int h = o / D, j = o % D;
      float sum = 0.0f;
#pragma unroll
      for (int g = 0; g < TS; ++g) sum += red[(g * HB + h) * D + j];
      dst[((hq0 + h) * p.n_splits + split) * D + j] = sum;
    }
    __syncthreads();
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
  // unrolled by eight so that eight splits' loads are in flight at once
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, ml[(bh * p.n_splits + s) * 2]);
  float L = 0.0f, rot = 0.0f, plain = 0.0f;
  if (M != -INFINITY) {
#pragma unroll 8
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

template <int D, int GW, int TT>
void launch_hb(int hb, dim3 grid, size_t smem, hipStream_t stream, const DecodeParams &p) {
  switch (hb) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, GW, 1, TT>), grid, dim3(kBlock), smem, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, GW, 2, TT>), grid, dim3(kBlock), smem, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, GW, 4, TT>), grid, dim3(kBlock), smem, stream, p); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, GW, 8, TT>), grid, dim3(kBlock), smem, stream, p); break;
  }
}

template <int D>
hipError_t launch_d(const DecodeParams &p, hipStream_t stream) {
  const RefLayout L32 = ref_layout(p, D, 32);
  auto a16 = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
  const bool vec = L32.kw % 4 == 0 && L32.vw_cold % 4 == 0 && L32.vw_hot % 4 == 0 && a16(p.k.codes) &&
                   a16(p.k.fp16) && a16(p.v.codes) && a16(p.v.fp16);
  // 64-position tiles when their 16-byte pieces fit four per lane
  const int vmax = L32.vw_cold > L32.vw_hot ? L32.vw_cold : L32.vw_hot;
  const bool t64 = vec && 64 * (L32.kw / 4 + vmax / 4) <= 4 * kBlock;
  const RefLayout L = t64 ? ref_layout(p, D, 64) : L32;
  const size_t smem = sizeof(uint32_t) * static_cast<size_t>(L.total);
  const dim3 grid(p.n_splits, p.batch * p.kv_heads, L.ngroups);
  if (t64) {
    launch_hb<D, 4, 64>(L.hb, grid, smem, stream, p);
  } else if (vec) {
    launch_hb<D, 4, 32>(L.hb, grid, smem, stream, p);
  } else {
    launch_hb<D, 1, 32>(L.hb, grid, smem, stream, p);
  }
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
