"""CPU oracle for TurboQuant KV-cache quantization and compressed-cache decode
attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP library (no kernels, headers, tables or helpers), and the
HIP library never imports, links or calls it.

Everything here is plain NumPy/SciPy in float64 and follows the method step
by step as the source pages describe it:

* "TurboQuant KV Cache Quantization in MLX-VLM" (mlx-vlm deep-dive page),
  sections "The TurboQuantKVCache Class" (packed uint32 words plus per-token
  norms, tensor shape kept), "Quantization Codecs and Bit Splitting"
  (floor(bits) to keys, ceil(bits) to values), "How TurboQuant KV Cache
  Quantization Works" (random Hadamard rotation, Beta-pdf Lloyd-Max codebook,
  MSE decoding, scores from the compressed form) and the FAQ entry on
  dequantization (rotation matrix plus codebooks back to float32).
* "How to Use TurboQuant with the MLX-VLM CLI", section "What Is TurboQuant?"
  (deterministic random rotation followed by codebook quantization).
* mlxcel "TurboQuant KV cache" page, sections "Available modes" (fp16-K with
  TurboQuant V, and the delegated hot/cold V split) and "WHT head-dimension
  constraint" (power-of-two head dimension, no padding).

Readings taken where the pages are silent (each is also listed with the
design notes of the repository):

* Signs of the rotation come from SplitMix64 (Steele, Lea and Flood, 2014):
  sign j is negative when the top bit of output j is set.
* Rotation R = H_d diag(s) / sqrt(d) with H_d the Sylvester (natural order)
  Hadamard matrix; one rotation per cache, shared by K and V.
* The "Beta-shaped" pdf is the exact marginal of one coordinate of a uniform
  unit vector in R^d: f_d(x) proportional to (1 - x^2)^((d - 3) / 2).
* The codebook is the Lloyd-Max fixed point of f_d with 2^b levels.  The pdf
  is symmetric, so the codebook is antisymmetric; the positive half is
  iterated and mirrored, which puts the middle threshold at exactly 0.
* Code j of a row = number of thresholds strictly below y_j (ties go to the
  lower code).  A zero row has norm 0, y = 0 and every code L/2 - 1.
* Codes are packed LSB-first as one bitstream per row: code j occupies bits
  [b*j, b*j + b) of the row; word w holds bits [32 w, 32 w + 32).
* Norms are stored as float32, one per (token, head).
* Decode: scale 1/sqrt(d), query head h reads KV head floor(h / G), no mask.
* Delegated V: the newest ``hot`` tokens are kept fp16 in a ring indexed by
  position mod ``hot``; an evicted token is quantized into the packed cold
  store at its own position.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy.special import betainc, betaincinv, gammaln

MASK64 = (1 << 64) - 1

__all__ = [
    "splitmix64", "sign_vector", "sylvester_hadamard", "rotation_matrix",
    "coord_pdf", "coord_tail", "cell_mass", "cell_first_moment",
    "cell_second_moment", "lloyd_max", "distortion", "split_bits",
    "row_words", "bytes_per_token_head", "quantize", "pack_codes",
    "unpack_codes", "codes_from_rotated", "dequantize", "attention", "PackedSide", "DelegatedSide",
    "decode_attention", "sparse_v_bound", "sparse_v_attention",
    "int8_quantize", "int8_levels", "int8_dequantize", "int8_bytes_per_token_head",
]


# ---------------------------------------------------------------------------
# Rotation: seeded sign-diagonal Walsh-Hadamard transform
# ("How TurboQuant KV Cache Quantization Works": random Hadamard transform;
#  CLI guide "What Is TurboQuant?": deterministic random rotation)
# ---------------------------------------------------------------------------

def splitmix64(seed: int, n: int) -> list[int]:
    """First ``n`` outputs of SplitMix64 started from ``seed``.

    Published generator (Steele, Lea and Flood, OOPSLA 2014): the state moves
    by the golden-ratio increment and each output is the state passed through
    two xor-shift-multiply rounds and a final xor-shift.
    """
    out = []
    state = seed & MASK64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_vector(seed: int, d: int) -> np.ndarray:
    """s_j = -1 if the top bit of SplitMix64 output j is set, else +1."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64(seed, d)])


def sylvester_hadamard(d: int) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j), natural (Sylvester) order, int64."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(d)
    pc = np.zeros((d, d), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        pc += a & 1
        a = a >> 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rotation_matrix(seed: int, d: int) -> np.ndarray:
    """R = H_d diag(s) / sqrt(d) (orthogonal, float64)."""
    return sylvester_hadamard(d).astype(np.float64) * sign_vector(seed, d)[None, :] / math.sqrt(d)


# ---------------------------------------------------------------------------
# The coordinate pdf and the Lloyd-Max codebook
# ("How TurboQuant KV Cache Quantization Works": Beta-pdf Lloyd-Max quantizer;
#  "Quantization Codecs and Bit Splitting": one MSE codec per side)
# ---------------------------------------------------------------------------

def _log_norm_const(d: int) -> float:
    """log C_d with f_d(x) = C_d (1 - x^2)^((d - 3)/2) on [-1, 1]."""
    return gammaln(d / 2.0) - gammaln((d - 1) / 2.0) - 0.5 * math.log(math.pi)


def coord_pdf(x, d: int):
    """Density of one coordinate of a uniform unit vector in R^d."""
    x = np.asarray(x, dtype=np.float64)
    return np.exp(_log_norm_const(d)) * (1.0 - x * x) ** ((d - 3) / 2.0)


def coord_tail(t, d: int):
    """P(X > t).  (1 + X)/2 is Beta((d-1)/2, (d-1)/2), so P(X > t) is the
    regularized incomplete beta function at (1 - t)/2."""
    a = (d - 1) / 2.0
    t = np.asarray(t, dtype=np.float64)
    return betainc(a, a, (1.0 - t) / 2.0)


def cell_mass(lo, hi, d: int):
    """P(lo < X <= hi) as a difference of upper tails; a cell on the negative
    side is mirrored first (the pdf is even) so that small tail masses are not
    taken as a difference of two numbers close to 1."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    neg = hi <= 0.0
    return np.where(neg, coord_tail(-hi, d) - coord_tail(-lo, d),
                    coord_tail(lo, d) - coord_tail(hi, d))


def cell_first_moment(lo, hi, d: int):
    """Integral of x f_d(x) over [lo, hi], closed form:
    C_d / (d - 1) * [(1 - lo^2)^((d-1)/2) - (1 - hi^2)^((d-1)/2)]."""
    return _first_moment_antiderivative(lo, d) - _first_moment_antiderivative(hi, d)


def _first_moment_antiderivative(x, d: int):
    """F1(x) = C_d (1 - x^2)^((d-1)/2) / (d - 1); d/dx F1 = -x f_d(x)."""
    x = np.asarray(x, dtype=np.float64)
    return np.exp(_log_norm_const(d)) / (d - 1) * (1.0 - x * x) ** ((d - 1) / 2.0)


def cell_second_moment(lo, hi, d: int):
    """Integral of x^2 f_d(x) over [lo, hi].

    Integration by parts with u = x, dv = x f_d dx gives
    lo F1(lo) - hi F1(hi) + (1/(d - 1)) C_d / C_{d+2} * mass_{d+2}, and
    C_d / C_{d+2} = (d - 1)/d, so the last term is mass_{d+2}(lo, hi) / d.
    """
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    return (lo * _first_moment_antiderivative(lo, d)
            - hi * _first_moment_antiderivative(hi, d)
            + cell_mass(lo, hi, d + 2) / d)


@functools.lru_cache(maxsize=None)
def _lloyd_max_cached(d: int, bits: int, tol: float, max_iter: int, stall: int):
    return _lloyd_max(d, bits, tol, max_iter, stall)


def lloyd_max(d: int, bits: int, tol: float = 1e-13, max_iter: int = 1000000,
              stall: int = 2000):
    """Lloyd-Max codebook of f_d with 2^bits levels (cached; returns copies).

    See :func:`_lloyd_max` for the iteration."""
    c, t = _lloyd_max_cached(int(d), int(bits), float(tol), int(max_iter), int(stall))
    return c.copy(), t.copy()


def _lloyd_max(d: int, bits: int, tol: float, max_iter: int, stall: int):
    """Lloyd-Max codebook of f_d with L = 2^bits levels.

    Returns (centroids[L] ascending, thresholds[L-1]) in float64.

    The positive half is iterated: cell edges e_0 = 0, e_i = midpoint of
    centroids i-1 and i, e_h = 1; each centroid is the conditional mean of its
    cell.  Start: centroid i at the CDF quantile (h + i + 1/2) / L.  Stop when
    no centroid moves by more than ``tol`` times the largest centroid, or when
    the largest movement has not reached a new minimum for ``stall`` steps
    (the float64 rounding floor of the cell integrals), or after ``max_iter``
    steps.  The full codebook is the mirror image (c_k = -c_{L-1-k});
    thresholds are the midpoints, the middle one exactly 0.
    """
    if bits < 1:
        raise ValueError("bits must be >= 1")
    L = 1 << bits
    h = L // 2
    a = (d - 1) / 2.0
    probs = (h + np.arange(h) + 0.5) / L
    p = 2.0 * betaincinv(a, a, probs) - 1.0
    best, since = np.inf, 0
    for _ in range(max_iter):
        edges = np.concatenate(([0.0], 0.5 * (p[:-1] + p[1:]), [1.0]))
        new = cell_first_moment(edges[:-1], edges[1:], d) / cell_mass(edges[:-1], edges[1:], d)
        moved = np.max(np.abs(new - p))
        p = new
        if moved <= tol * np.max(np.abs(p)):
            break
        if moved < best:
            best, since = moved, 0
        else:
            since += 1
            if since >= stall:
                break
    centroids = np.concatenate((-p[::-1], p))
    thresholds = 0.5 * (centroids[:-1] + centroids[1:])
    thresholds[h - 1] = 0.0
    return centroids, thresholds


def distortion(d: int, centroids, thresholds) -> float:
    """E[(X - Q(X))^2] for X ~ f_d, by the definition summed cell by cell."""
    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate(([-1.0], np.asarray(thresholds, np.float64), [1.0]))
    lo, hi = edges[:-1], edges[1:]
    return float(np.sum(cell_second_moment(lo, hi, d)
                        - 2.0 * c * cell_first_moment(lo, hi, d)
                        + c * c * cell_mass(lo, hi, d)))


# ---------------------------------------------------------------------------
# Bit budget and storage ("Quantization Codecs and Bit Splitting";
# "The TurboQuantKVCache Class": packed uint32 words plus per-token norms)
# ---------------------------------------------------------------------------

def split_bits(bits: float) -> tuple[int, int]:
    """Keys get floor(bits), values get ceil(bits)."""
    return int(math.floor(bits)), int(math.ceil(bits))


def row_words(d: int, bits: int) -> int:
    """uint32 words per packed row: ceil(bits * d / 32)."""
    return (bits * d + 31) // 32


def bytes_per_token_head(d: int, bits: int) -> int:
    """Packed bytes per (token, head) of one side: words plus a float32 norm."""
    return 4 * row_words(d, bits) + 4


# ---------------------------------------------------------------------------
# Quantize / pack / dequantize (MSE codec on the rotated unit vector)
# ---------------------------------------------------------------------------

def quantize(x, R, thresholds, chunk: int = 4096):
    """Quantize rows of ``x`` (float16 [..., d]).

    Returns (codes int64 [..., d], norms float64 [...], y float64 [..., d])
    with n = ||x||, u = x / n (u = 0 when n = 0), y = R u and
    code_j = #{k : y_j > t_k}.
    """
    x = np.asarray(x)
    shape = x.shape
    d = shape[-1]
    xf = x.reshape(-1, d).astype(np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    n = np.sqrt(np.sum(xf * xf, axis=1))
    safe = np.where(n > 0.0, n, 1.0)
    u = np.where(n[:, None] > 0.0, xf / safe[:, None], 0.0)
    y = u @ R.T
    codes = codes_from_rotated(y, t, chunk)
    return codes.reshape(shape), n.reshape(shape[:-1]), y.reshape(shape)


def codes_from_rotated(y, thresholds, chunk: int = 4096) -> np.ndarray:
    """code = #{k : y > t_k} for every element of ``y`` (any shape)."""
    y = np.asarray(y, dtype=np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    flat = y.reshape(-1)
    codes = np.empty(flat.shape, dtype=np.int64)
    for s in range(0, flat.size, chunk * 64):
        yy = flat[s:s + chunk * 64]
        codes[s:s + chunk * 64] = np.sum(yy[:, None] > t[None, :], axis=1)
    return codes.reshape(y.shape)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack rows of codes LSB-first into uint32 words [..., W]."""
    codes = np.asarray(codes, dtype=np.int64)
    shape = codes.shape
    d = shape[-1]
    W = row_words(d, bits)
    flat = codes.reshape(-1, d)
    if np.any(flat < 0) or np.any(flat >= (1 << bits)):
        raise ValueError("code out of range")
    # bit r of code j is stream bit b*j + r
    stream = ((flat[:, :, None] >> np.arange(bits)[None, None, :]) & 1).reshape(flat.shape[0], d * bits)
    pad = W * 32 - d * bits
    if pad:
        stream = np.concatenate([stream, np.zeros((flat.shape[0], pad), np.int64)], axis=1)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    words = (stream.reshape(-1, W, 32).astype(np.uint64) * weights).sum(axis=2)
    return words.astype(np.uint32).reshape(shape[:-1] + (W,))


def unpack_codes(words, bits: int, d: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: words [..., W] -> codes [..., d]."""
    words = np.asarray(words, dtype=np.uint32)
    shape = words.shape
    W = shape[-1]
    flat = words.reshape(-1, W).astype(np.uint64)
    stream = ((flat[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).reshape(flat.shape[0], W * 32)
    stream = stream[:, : d * bits].reshape(-1, d, bits).astype(np.int64)
    codes = (stream << np.arange(bits)[None, None, :]).sum(axis=2)
    return codes.reshape(shape[:-1] + (d,))


def dequantize(codes, norms, R, centroids) -> np.ndarray:
    """x~ = n * R^T c[code] (float64 [..., d])."""
    c = np.asarray(centroids, dtype=np.float64)[np.asarray(codes)]
    return np.asarray(norms, dtype=np.float64)[..., None] * (c @ R)


# ---------------------------------------------------------------------------
# Attention by its plain definition (decode: one query token per sequence)
# ---------------------------------------------------------------------------

def attention(q, k, v):
    """q [B, Hq, d]; k, v [B, Hkv, T, d] (float64 after widening).

    Query head h uses KV head floor(h / G), G = Hq / Hkv.  Returns
    (out [B, Hq, d], scores [B, Hq, T]) with scores = q.k / sqrt(d) and
    out = softmax(scores) @ v.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    T = k.shape[2]
    out = np.zeros((B, Hq, d))
    scores = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            s = k[b, kv] @ q[b, h] / math.sqrt(d)
            p = np.exp(s - np.max(s)) if T else s
            p = p / np.sum(p) if T else p
            scores[b, h] = s
            out[b, h] = p @ v[b, kv] if T else 0.0
    return out, scores


def sparse_v_bound(q, k, v, tau):
    """Sparse-V (mlxcel "TurboQuant KV cache", "CLI and server flags": a
    weight threshold below which value work is skipped, 0 disabling it).
    With p_i = exp(s_i - max s) the weights relative to the largest, a
    decode that drops the value contribution of some positions with
    p_i < tau, keeping every p_i in the denominator, moves output element j
    by at most  sum_{i: p_i < tau} p_i |v_ij| / sum_i p_i.  Returns that
    bound [B, Hq, d] (zero for tau = 0)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    bound = np.zeros((B, Hq, d))
    if k.shape[2] == 0:
        return bound
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            s = k[b, kv] @ q[b, h] / math.sqrt(d)
            p = np.exp(s - np.max(s))
            low = p < tau
            bound[b, h] = (p[low] @ np.abs(v[b, kv][low])) / np.sum(p)
    return bound


def sparse_v_attention(q, k, v, tau):
    """Attention that drops the value contribution of every position with
    p_i < tau (relative weight, as in sparse_v_bound) and keeps all of them
    in the softmax denominator: the largest drop the bound allows."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((B, Hq, d))
    if k.shape[2] == 0:
        return out
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            s = k[b, kv] @ q[b, h] / math.sqrt(d)
            p = np.exp(s - np.max(s))
            keep = ~(p < tau)
            out[b, h] = (p[keep] @ v[b, kv][keep]) / np.sum(p)
    return out


# ---------------------------------------------------------------------------
# INT8 per-token absmax cache (mlxcel "TurboQuant KV cache", "Available
# modes": int8 is per-token INT8 absmax quantization, ~2x)
# ---------------------------------------------------------------------------

def int8_levels(x):
    """The quantity each INT8 code rounds: v_j = 127 x_j / max_i |x_i| per
    row, in float64 (0 for a zero row).  fp16 inputs are exact in float64,
    127 x_j is exact, and the one rounding of the division cannot move v
    across a half-integer: v is a ratio of fp16 multiples whose distance from
    any half-integer, when not zero, is far above the float64 rounding."""
    x64 = np.asarray(x).astype(np.float64)
    a = np.max(np.abs(x64), axis=-1)
    safe = np.where(a > 0, a, 1.0)
    return np.where(a[..., None] > 0, 127.0 * x64 / safe[..., None], 0.0)


def int8_quantize(x):
    """Per row (one token of one head): a = max_j |x_j|, code_j = the integer
    nearest to 127 x_j / a (ties to even), which lies in [-127, 127] by
    construction; the stored scale is a / 127 rounded to float32 (the
    storage format keeps a float32 scale, and the dequantized row is code x
    scale).  A zero row has scale 0 and codes 0.  The decision is the exact
    definition, taken in float64 (see ``int8_levels``).  Returns (codes int8
    [..., d], scales float32 [...])."""
    x64 = np.asarray(x).astype(np.float64)
    a = np.max(np.abs(x64), axis=-1)
    codes = np.rint(int8_levels(x)).astype(np.int8)
    scale = (a / 127.0).astype(np.float32)
    return codes, scale


def int8_dequantize(codes, scales):
    """codes x scale, in float64."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scales).astype(np.float64)[..., None]


def int8_bytes_per_token_head(d: int) -> int:
    """One byte per coordinate plus a float32 scale."""
    return d + 4


# ---------------------------------------------------------------------------
# Cache sides and their append bookkeeping
# ---------------------------------------------------------------------------

class PackedSide:
    """One packed side of a cache: codes [B, H, cap, d] and norms (kept as
    float32, as stored).  Rows outside an append stay untouched."""

    def __init__(self, batch, heads, capacity, d, bits, seed):
        self.bits = bits
        self.d = d
        self.R = rotation_matrix(seed, d)
        self.centroids, self.thresholds = lloyd_max(d, bits)
        self.codes = np.zeros((batch, heads, capacity, d), np.int64)
        self.norms = np.zeros((batch, heads, capacity), np.float32)

    def write(self, x, pos):
        """Quantize x [B, H, n, d] into rows pos .. pos + n - 1."""
        codes, n, _ = quantize(x, self.R, self.thresholds)
        self.codes[:, :, pos:pos + x.shape[2]] = codes
        self.norms[:, :, pos:pos + x.shape[2]] = n.astype(np.float32)

    def rows(self, start, count):
        return dequantize(self.codes[:, :, start:start + count],
                          self.norms[:, :, start:start + count].astype(np.float64),
                          self.R, self.centroids)


class DelegatedSide:
    """Delegated V: newest ``hot`` tokens fp16 in a ring (slot = position mod
    hot); older tokens packed in a cold store at their own positions."""

    def __init__(self, batch, heads, capacity, d, bits, seed, hot):
        self.hot = hot
        self.cold = PackedSide(batch, heads, capacity, d, bits, seed)
        self.ring = np.zeros((batch, heads, hot, d), np.float16)

    def append(self, x, offset):
        """Append x [B, H, n, d] at positions offset .. offset + n - 1, one
        position at a time: the ring slot's previous occupant (position
        p - hot) is quantized into the cold store, then the slot is
        overwritten."""
        for i in range(x.shape[2]):
            p = offset + i
            slot = p % self.hot
            if p >= self.hot:
                self.cold.write(self.ring[:, :, slot:slot + 1], p - self.hot)
            self.ring[:, :, slot] = x[:, :, i]

    def rows(self, length):
        """Float64 V rows 0 .. length - 1 as the decode step sees them."""
        B, H, _, d = self.ring.shape
        out = np.zeros((B, H, length, d))
        n_cold = max(0, length - self.hot)
        if n_cold:
            out[:, :, :n_cold] = self.cold.rows(0, n_cold)
        for p in range(n_cold, length):
            out[:, :, p] = self.ring[:, :, p % self.hot].astype(np.float64)
        return out


def decode_attention(q, k_rows, v_rows):
    """Decode step over dense float64 K/V rows (already dequantized or
    widened from fp16).  Returns (out, scores) from :func:`attention`."""
    return attention(q, k_rows, v_rows)
