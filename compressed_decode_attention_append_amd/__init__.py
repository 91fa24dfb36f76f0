"""Python binding of libtq (TurboQuant KV-cache quantize-append and decode
attention from the packed cache, MI355X / gfx950).

Argument marshalling only: every step of the path runs in libtq's HIP
kernels; torch provides device memory and the current HIP stream.  The
functions keep the names of the C ABI in ``include/tq.h``.  If ``libtq.so``
has not been built, importing succeeds but every call raises ``TQError``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_ARG = -1
TQ_ERR_HEAD_DIM = -2
TQ_ERR_BITS = -3
TQ_ERR_CAPACITY = -4
TQ_ERR_WORKSPACE = -5
TQ_ERR_MODE = -6
TQ_ERR_HIP = -7
TQ_ERR_SCRATCH = -8

SIDE_FP16 = 0
SIDE_PACKED = 1
SIDE_DELEGATED = 2
SIDE_INT8 = 3
_MODES = {"fp16": SIDE_FP16, "packed": SIDE_PACKED, "delegated": SIDE_DELEGATED, "int8": SIDE_INT8}


class TQError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = None):
        self.status = status
        super().__init__(f"{what}: {detail if detail is not None else status_string(status)} ({status})")


class tq_side(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int),
        ("bits", ctypes.c_int),
        ("centroids", ctypes.c_void_p),
        ("thresholds", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("norms", ctypes.c_void_p),
        ("fp16", ctypes.c_void_p),
        ("hot", ctypes.c_int),
    ]


class tq_cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int),
        ("kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("capacity", ctypes.c_int),
        ("seed", ctypes.c_uint64),
        ("k", tq_side),
        ("v", tq_side),
        ("block_table", ctypes.c_void_p),
        ("block_size", ctypes.c_int),
        ("max_blocks", ctypes.c_int),
        ("num_blocks", ctypes.c_int),
    ]


_lib = None


def lib():
    """The loaded libtq (raises TQError if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TQError(TQ_ERR_HIP, f"libtq.so is not built at {LIB_PATH}", "libtq not built")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.tq_split_bits.argtypes = [ctypes.c_double, ctypes.POINTER(I), ctypes.POINTER(I)]
        L.tq_split_bits.restype = I
        L.tq_row_words.argtypes = [I, I]
        L.tq_row_words.restype = I
        L.tq_sign_words.argtypes = [ctypes.c_uint64, I, P]
        L.tq_sign_words.restype = I
        L.tq_build_codebook.argtypes = [I, I, P, P]
        L.tq_build_codebook.restype = I
        L.tq_quantize_append.argtypes = [ctypes.POINTER(tq_cache), P, P, I, I, P]
        L.tq_quantize_append.restype = I
        L.tq_decode_workspace_bytes.argtypes = [ctypes.POINTER(tq_cache), I, I, I]
        L.tq_decode_workspace_bytes.restype = ctypes.c_size_t
        L.tq_decode_workspace_init.argtypes = [P, ctypes.c_size_t, P]
        L.tq_decode_workspace_init.restype = I
        L.tq_decode_attention.argtypes = [ctypes.POINTER(tq_cache), P, I, I, I, P, P, P,
                                          ctypes.c_size_t, P]
        L.tq_decode_attention.restype = I
        L.tq_decode_attention_sparse.argtypes = [ctypes.POINTER(tq_cache), P, I, I, I, ctypes.c_float, P, P,
                                                 P, ctypes.c_size_t, P]
        L.tq_decode_attention_sparse.restype = I
        L.tq_decode_attention_append.argtypes = [ctypes.POINTER(tq_cache), P, P, I, P, I, I, I, P, P, P,
                                                 ctypes.c_size_t, P]
        L.tq_decode_attention_append.restype = I
        L.tq_decode_attention_noalloc.argtypes = [ctypes.POINTER(tq_cache), P, I, I, I, P, P, P]
        L.tq_decode_attention_noalloc.restype = I
        L.tq_dequantize.argtypes = [ctypes.POINTER(tq_cache), I, I, I, P, P]
        L.tq_dequantize.restype = I
        L.tq_status_string.argtypes = [I]
        L.tq_status_string.restype = ctypes.c_char_p
        L.tq_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
        L.tq_read_probe.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().tq_status_string(int(status)).decode()
    except TQError:
        return "libtq not built"


def _check(status: int, what: str):
    if status != TQ_OK:
        raise TQError(status, what)


def split_bits(bits: float) -> tuple[int, int]:
    k, v = ctypes.c_int(), ctypes.c_int()
    _check(lib().tq_split_bits(float(bits), ctypes.byref(k), ctypes.byref(v)), "tq_split_bits")
    return k.value, v.value


def row_words(head_dim: int, bits: int) -> int:
    r = lib().tq_row_words(int(head_dim), int(bits))
    if r < 0:
        raise TQError(r, "tq_row_words")
    return r


def sign_words(seed: int, head_dim: int) -> np.ndarray:
    out = np.zeros(max(1, head_dim // 32), np.uint32)
    _check(lib().tq_sign_words(int(seed), int(head_dim), out.ctypes.data), "tq_sign_words")
    return out


def build_codebook(head_dim: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Lloyd-Max codebook (float64 centroids[2^bits], thresholds[2^bits - 1])."""
    L = 1 << int(bits) if 1 <= int(bits) <= 8 else 2
    c = np.zeros(L, np.float64)
    t = np.zeros(L - 1, np.float64)
    _check(lib().tq_build_codebook(int(head_dim), int(bits), c.ctypes.data, t.ctypes.data),
           "tq_build_codebook")
    return c, t


_CODEBOOKS: dict = {}


class Codebook:
    """Host codebook of one (head_dim, bits), built once by tq_build_codebook
    and kept as the fp32 arrays the cache descriptor points at."""

    def __init__(self, head_dim: int, bits: int):
        self.head_dim, self.bits = int(head_dim), int(bits)
        self.centroids64, self.thresholds64 = build_codebook(head_dim, bits)
        self.centroids = np.ascontiguousarray(self.centroids64.astype(np.float32))
        self.thresholds = np.ascontiguousarray(self.thresholds64.astype(np.float32))

    @classmethod
    def get(cls, head_dim: int, bits: int) -> "Codebook":
        key = (int(head_dim), int(bits))
        if key not in _CODEBOOKS:
            _CODEBOOKS[key] = cls(*key)
        return _CODEBOOKS[key]


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


WORKSPACE_COUNTER_BYTES = 256 * 1024
TQ_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


def decode_workspace_init(workspace, stream=None) -> None:
    """Zero the counter region of a device workspace tensor (tq.h:
    tq_decode_workspace_init); needed once before its first decode."""
    _check(lib().tq_decode_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream_handle(stream)), "tq_decode_workspace_init")


def read_probe(buf, sink, stream=None) -> None:
    """Stream-read the device tensor `buf` (a multiple of 16 bytes, 16-byte
    aligned) with the library's probe kernel and write the xor of its 32-bit
    words to the 1-element int32/uint32 device tensor `sink`.  A measurement
    aid for the attainable HBM read bandwidth, not part of the method."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().tq_read_probe(_ptr(buf) if nbytes else None, nbytes, _ptr(sink), _stream_handle(stream)),
           "tq_read_probe")


@dataclass
class SideSpec:
    mode: str = "packed"   # "fp16" | "packed" | "delegated"
    bits: int = 4
    hot: int = 256


class TQCache:
    """One layer's cache in device memory plus its C descriptor.

    Layouts (all contiguous): codes [B][Hkv][cap][W] int32 (uint32 bits),
    norms [B][Hkv][cap] fp32, fp16 rows [B][Hkv][cap][d], delegated ring
    [B][Hkv][hot][d].  Buffers start zeroed.
    """

    def __init__(self, batch, kv_heads, head_dim, capacity, k: SideSpec, v: SideSpec,
                 seed: int = 0, device="cuda", block_table=None, block_size: int = 0,
                 num_blocks: int = 0):
        """Contiguous sides by default.  Paged: ``block_table`` is an int32
        [B][capacity / block_size] tensor of block indices (kept on the
        device), and the sides are pools of ``num_blocks`` blocks
        ([num_blocks][Hkv][block_size][...]); see tq_cache in tq.h."""
        import torch
        self.batch, self.kv_heads, self.head_dim = int(batch), int(kv_heads), int(head_dim)
        self.capacity, self.seed = int(capacity), int(seed)
        self.k_spec, self.v_spec = k, v
        self.device = device
        self._keep = []
        self.desc = tq_cache()
        self.desc.batch, self.desc.kv_heads = self.batch, self.kv_heads
        self.desc.head_dim, self.desc.capacity = self.head_dim, self.capacity
        self.desc.seed = self.seed
        self.tensors = {}
        self.paged = block_table is not None
        if self.paged:
            bs = int(block_size)
            if bs <= 0 or self.capacity % bs:
                raise ValueError("paged cache: capacity must be a multiple of block_size")
            if tuple(block_table.shape) != (self.batch, self.capacity // bs):
                raise ValueError(f"block_table must be [{self.batch}][{self.capacity // bs}]")
            if int(num_blocks) < 1:
                raise ValueError("paged cache: num_blocks must be at least 1")
            # the table is at hand here, so its entries are range-checked on
            # the host (the library itself only guards them on the device)
            host = block_table.detach().to("cpu", torch.int64)
            if host.numel() and (int(host.min()) < 0 or int(host.max()) >= int(num_blocks)):
                raise ValueError(f"block_table entries must lie in [0, {int(num_blocks)})")
            table = block_table.to(device=device, dtype=torch.int32).contiguous()
            self.block_table, self.block_size, self.num_blocks = table, bs, int(num_blocks)
            self.desc.block_table = _ptr(table)
            self.desc.block_size, self.desc.max_blocks = bs, self.capacity // bs
            self.desc.num_blocks = self.num_blocks
        for name, spec, side in (("k", k, self.desc.k), ("v", v, self.desc.v)):
            side.mode = _MODES[spec.mode]
            side.bits = int(spec.bits) if spec.mode in ("packed", "delegated") else 0
            side.hot = int(spec.hot) if spec.mode == "delegated" else 0
            B, H, cap, d = self.batch, self.kv_heads, self.capacity, self.head_dim
            if self.paged:
                # pools: [num_blocks][Hkv][block_size][...] in the same tensor
                # shapes (B -> num_blocks, cap -> block_size)
                B, cap = self.num_blocks, self.block_size
            if spec.mode in ("packed", "delegated"):
                cb = Codebook.get(d, spec.bits)
                self._keep.append(cb)
                side.centroids = cb.centroids.ctypes.data
                side.thresholds = cb.thresholds.ctypes.data
                W = row_words(d, spec.bits)
                codes = torch.zeros((B, H, cap, W), dtype=torch.int32, device=device)
                norms = torch.zeros((B, H, cap), dtype=torch.float32, device=device)
                side.codes, side.norms = _ptr(codes), _ptr(norms)
                self.tensors[name + "_codes"] = codes
                self.tensors[name + "_norms"] = norms
            if spec.mode == "int8":
                # codes: d int8 a row as d / 4 words; norms: the per-row scale
                codes = torch.zeros((B, H, cap, d // 4), dtype=torch.int32, device=device)
                norms = torch.zeros((B, H, cap), dtype=torch.float32, device=device)
                side.codes, side.norms = _ptr(codes), _ptr(norms)
                self.tensors[name + "_codes"] = codes
                self.tensors[name + "_norms"] = norms
            if spec.mode == "fp16":
                rows = torch.zeros((B, H, cap, d), dtype=torch.float16, device=device)
                side.fp16 = _ptr(rows)
                self.tensors[name + "_fp16"] = rows
            if spec.mode == "delegated":
                ring = torch.zeros((self.batch, H, spec.hot, d), dtype=torch.float16, device=device)
                side.fp16 = _ptr(ring)
                self.tensors[name + "_ring"] = ring
        self._ws = None

    # -- the four operations ------------------------------------------------
    def quantize_append(self, k_new, v_new, offset: int, stream=None):
        """k_new, v_new: fp16 [B][Hkv][n][d] on the device."""
        for x in (k_new, v_new):
            self._check_rows(x)
        n = int(k_new.shape[2])
        if int(v_new.shape[2]) != n:
            raise ValueError("k_new and v_new differ in length")
        _check(lib().tq_quantize_append(ctypes.byref(self.desc), _ptr(k_new), _ptr(v_new), n,
                                        int(offset), _stream_handle(stream)),
               "tq_quantize_append")

    def workspace_bytes(self, q_heads: int, length: int, n_splits: int = 0) -> int:
        return int(lib().tq_decode_workspace_bytes(ctypes.byref(self.desc), int(q_heads),
                                                   int(length), int(n_splits)))

    def workspace(self, q_heads: int, length: int, n_splits: int = 0):
        import torch
        need = self.workspace_bytes(q_heads, length, n_splits)
        if need == 0:
            raise TQError(TQ_ERR_ARG, "tq_decode_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            decode_workspace_init(self._ws)
        return self._ws

    def decode_attention(self, q, length: int, n_splits: int = 0, out=None, scores=False,
                         workspace=None, stream=None, sparse_v: float = 0.0):
        """q: fp16 [B][Hq][d].  Returns out fp32 [B][Hq][d] (and scores
        fp32 [B][Hq][length] when ``scores`` is true).  ``sparse_v`` > 0 runs
        tq_decode_attention_sparse with that threshold."""
        import torch
        if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 3:
            raise ValueError("q must be contiguous fp16 [B, Hq, d]")
        B, Hq, d = q.shape
        if B != self.batch or d != self.head_dim:
            raise ValueError("q shape does not match the cache")
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        sc = torch.empty((B, Hq, max(int(length), 1)), dtype=torch.float32, device=q.device) if scores else None
        ws = workspace if workspace is not None else self.workspace(Hq, length, n_splits)
        if sparse_v:
            _check(lib().tq_decode_attention_sparse(ctypes.byref(self.desc), _ptr(q), int(Hq), int(length),
                                                    int(n_splits), float(sparse_v), _ptr(out), _ptr(sc),
                                                    _ptr(ws), ws.numel() * ws.element_size(),
                                                    _stream_handle(stream)),
                   "tq_decode_attention_sparse")
        else:
            _check(lib().tq_decode_attention(ctypes.byref(self.desc), _ptr(q), int(Hq), int(length),
                                             int(n_splits), _ptr(out), _ptr(sc), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream_handle(stream)),
                   "tq_decode_attention")
        return (out, sc[:, :, :length]) if scores else out

    def decode_attention_append(self, k_new, v_new, offset: int, q, length: int, n_splits: int = 0, out=None,
                                scores=False, workspace=None, stream=None):
        """One decode step's append-then-attend through
        tq_decode_attention_append: the new position k_new, v_new (fp16
        [B, Hkv, 1, d]) written at row `offset`, then attention over
        [0, length).  Returns what decode_attention returns."""
        import torch
        for x in (k_new, v_new):
            self._check_rows(x)
        if int(k_new.shape[2]) != 1 or int(v_new.shape[2]) != 1:
            raise ValueError("k_new and v_new hold one position")
        if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 3:
            raise ValueError("q must be contiguous fp16 [B, Hq, d]")
        B, Hq, d = q.shape
        if B != self.batch or d != self.head_dim:
            raise ValueError("q shape does not match the cache")
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        sc = torch.empty((B, Hq, max(int(length), 1)), dtype=torch.float32, device=q.device) if scores else None
        ws = workspace if workspace is not None else self.workspace(Hq, length, n_splits)
        _check(lib().tq_decode_attention_append(ctypes.byref(self.desc), _ptr(k_new), _ptr(v_new), int(offset),
                                                _ptr(q), int(Hq), int(length), int(n_splits), _ptr(out), _ptr(sc),
                                                _ptr(ws), ws.numel() * ws.element_size(), _stream_handle(stream)),
               "tq_decode_attention_append")
        return (out, sc[:, :, :length]) if scores else out

    def decode_attention_noalloc(self, q, length: int, n_splits: int = 0, out=None, scores=False, stream=None):
        """decode_attention through tq_decode_attention_noalloc: the library's
        fixed per-GPU scratch instead of a workspace (for callers that cannot
        allocate; overlapping calls on one GPU race)."""
        import torch
        if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 3:
            raise ValueError("q must be contiguous fp16 [B, Hq, d]")
        B, Hq, d = q.shape
        if B != self.batch or d != self.head_dim:
            raise ValueError("q shape does not match the cache")
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        sc = torch.empty((B, Hq, max(int(length), 1)), dtype=torch.float32, device=q.device) if scores else None
        _check(lib().tq_decode_attention_noalloc(ctypes.byref(self.desc), _ptr(q), int(Hq), int(length),
                                                 int(n_splits), _ptr(out), _ptr(sc), _stream_handle(stream)),
               "tq_decode_attention_noalloc")
        return (out, sc[:, :, :length]) if scores else out

    def dequantize(self, side: str, start: int, count: int, stream=None):
        import torch
        out = torch.empty((self.batch, self.kv_heads, max(int(count), 1), self.head_dim),
                          dtype=torch.float32, device=self.device)
        _check(lib().tq_dequantize(ctypes.byref(self.desc), 0 if side == "k" else 1, int(start),
                                   int(count), _ptr(out), _stream_handle(stream)),
               "tq_dequantize")
        return out[:, :, :count]

    def logical(self, name: str):
        """A side tensor in the logical [B][Hkv][capacity][...] layout: the
        tensor itself for a contiguous cache (and for the delegated ring); for
        a paged cache the pool gathered through the block table."""
        t = self.tensors[name]
        if not self.paged or name.endswith("_ring"):
            return t
        g = t[self.block_table.long()]          # [B][max_blocks][Hkv][bs][...]
        g = g.transpose(1, 2)                    # [B][Hkv][max_blocks][bs][...]
        return g.reshape(self.batch, self.kv_heads, self.capacity, *t.shape[3:])

    def _check_rows(self, x):
        import torch
        if x.dtype != torch.float16 or not x.is_contiguous() or x.dim() != 4:
            raise ValueError("new rows must be contiguous fp16 [B, Hkv, n, d]")
        if (x.shape[0], x.shape[1], x.shape[3]) != (self.batch, self.kv_heads, self.head_dim):
            raise ValueError("new rows do not match the cache shape")


__all__ = [
    "TQError", "tq_side", "tq_cache", "lib", "status_string", "split_bits", "row_words",
    "sign_words", "build_codebook", "Codebook", "SideSpec", "TQCache", "SIDE_FP16",
    "decode_workspace_init", "WORKSPACE_COUNTER_BYTES",
    "SIDE_PACKED", "SIDE_DELEGATED",
]
