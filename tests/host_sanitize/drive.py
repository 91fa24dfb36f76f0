"""Drive every entry point of a host-only libtq build (launchers stubbed to
report "no device") through ctypes: the helpers, the codebook builder over
head sizes and widths, every argument check, and valid calls of every side
mode, contiguous and paged, which run all host code up to the launch.  Run
under the sanitizers by tests/test_host_sanitize.py; prints "driven N calls"
on success."""
import ctypes
import sys

import numpy as np

OK, ARG, HEAD, BITS, CAP, WS, MODE, HIP, SCR = 0, -1, -2, -3, -4, -5, -6, -7, -8


class Side(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("bits", ctypes.c_int), ("centroids", ctypes.c_void_p),
                ("thresholds", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("fp16", ctypes.c_void_p), ("hot", ctypes.c_int)]


class Cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("capacity", ctypes.c_int), ("seed", ctypes.c_uint64), ("k", Side), ("v", Side),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int), ("max_blocks", ctypes.c_int),
                ("num_blocks", ctypes.c_int)]


def main(path):
    L = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.tq_build_codebook.argtypes = [I, I, P, P]
    L.tq_split_bits.argtypes = [ctypes.c_double, P, P]
    L.tq_sign_words.argtypes = [ctypes.c_uint64, I, P]
    L.tq_quantize_append.argtypes = [ctypes.POINTER(Cache), P, P, I, I, P]
    L.tq_decode_workspace_bytes.argtypes = [ctypes.POINTER(Cache), I, I, I]
    L.tq_decode_workspace_bytes.restype = ctypes.c_size_t
    L.tq_decode_attention.argtypes = [ctypes.POINTER(Cache), P, I, I, I, P, P, P, ctypes.c_size_t, P]
    L.tq_decode_attention_sparse.argtypes = [ctypes.POINTER(Cache), P, I, I, I, ctypes.c_float, P, P, P,
                                             ctypes.c_size_t, P]
    L.tq_decode_attention_noalloc.argtypes = [ctypes.POINTER(Cache), P, I, I, I, P, P, P]
    L.tq_decode_attention_append.argtypes = [ctypes.POINTER(Cache), P, P, I, P, I, I, I, P, P, P,
                                             ctypes.c_size_t, P]
    L.tq_decode_workspace_init.argtypes = [P, ctypes.c_size_t, P]
    L.tq_dequantize.argtypes = [ctypes.POINTER(Cache), I, I, I, P, P]
    L.tq_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
    L.tq_status_string.restype = ctypes.c_char_p
    n = 0

    def call(fn, *a):
        nonlocal n
        n += 1
        return fn(*a)

    for s in range(1, -10, -1):
        assert call(L.tq_status_string, s)
    kb, vb = ctypes.c_int(), ctypes.c_int()
    for bits in (0.5, 1, 3.5, 4.2, 8, 8.5, float("nan"), float("inf")):
        call(L.tq_split_bits, bits, ctypes.byref(kb), ctypes.byref(vb))
    assert call(L.tq_split_bits, 3.5, None, None) == ARG
    for d in (16, 32, 64, 96, 128, 256, 512):
        for b in (0, 1, 4, 8, 9):
            call(L.tq_row_words, d, b)
    sw = np.zeros(8, np.uint32)
    for d in (32, 64, 128, 256, 100):
        call(L.tq_sign_words, 12345, d, sw.ctypes.data)
    tables = {}
    for d in (2, 32, 64, 128, 256, 4096, 65536):
        for b in range(1, 6):
            c, t = np.zeros(1 << b), np.zeros((1 << b) - 1)
            assert call(L.tq_build_codebook, d, b, c.ctypes.data, t.ctypes.data) == OK
            tables[(d, b)] = (c.astype(np.float32), t.astype(np.float32))
    c, t = np.zeros(64), np.zeros(63)
    assert call(L.tq_build_codebook, 128, 6, c.ctypes.data, t.ctypes.data) == OK
    for d, b in ((3, 3), (128, 0), (128, 9), (100, 3)):
        assert call(L.tq_build_codebook, d, b, c.ctypes.data, t.ctypes.data) != OK

    buf = np.zeros(1 << 22, np.uint8)
    base = (buf.ctypes.data + 255) & ~255
    table = np.arange(64, dtype=np.int32)

    def desc(d=128, km=1, vm=1, kbits=3, vbits=4, cap=1024, B=2, H=4, hot=128, paged=False):
        cd = Cache()
        cd.batch, cd.kv_heads, cd.head_dim, cd.capacity, cd.seed = B, H, d, cap, 7
        for side, mode, bits in ((cd.k, km, kbits), (cd.v, vm, vbits)):
            side.mode, side.bits, side.hot = mode, bits, hot
            cb = tables.get((d, bits), tables[(128, 4)])
            side.centroids, side.thresholds = cb[0].ctypes.data, cb[1].ctypes.data
            side.codes, side.norms, side.fp16 = base, base + 4096, base + 8192
        if paged:
            cd.block_table, cd.block_size, cd.max_blocks, cd.num_blocks = table.ctypes.data, 64, cap // 64, 64
        return cd

    combos = [(1, 1, 3, 4), (1, 1, 4, 4), (0, 1, 0, 4), (0, 2, 0, 4), (0, 0, 0, 0), (3, 3, 0, 0),
              (1, 3, 3, 0), (3, 1, 0, 4), (1, 1, 2, 5), (2, 1, 3, 4), (7, 1, 3, 4), (1, 1, 0, 4), (1, 1, 3, 9)]
    ws_big = 1 << 21
    for d in (32, 64, 128, 256, 48):
        for km, vm, kbits, vbits in combos:
            for paged in (False, True):
                for Hq in (4, 8, 32, 6):
                    cd = desc(d, km, vm, kbits, vbits, paged=paged)
                    for length in (0, 1, 300, 1024, 1025):
                        need = call(L.tq_decode_workspace_bytes, ctypes.byref(cd), Hq, length, 0)
                        for ns in (0, 3):
                            call(L.tq_decode_attention, ctypes.byref(cd), base, Hq, length, ns, base, None, base,
                                 ws_big, None)
                        call(L.tq_decode_attention_sparse, ctypes.byref(cd), base, Hq, length, 0, 0.5, base, base,
                             base, max(need, 1), None)
                        call(L.tq_decode_attention_noalloc, ctypes.byref(cd), base, Hq, length, 0, base, None, None)
                        for off, sc in ((max(length - 1, 0), None), (length, None), (max(length - 1, 0), base)):
                            call(L.tq_decode_attention_append, ctypes.byref(cd), base, base, off, base, Hq, length, 0,
                                 base, sc, base, ws_big, None)
                    for n_new, off in ((0, 0), (1, 0), (16, 1000), (300, 5), (2000, 0), (-1, 0)):
                        call(L.tq_quantize_append, ctypes.byref(cd), base, base, n_new, off, None)
                    for side in (0, 1, 2):
                        call(L.tq_dequantize, ctypes.byref(cd), side, 10, 100, base, None)
    cd = desc()
    assert call(L.tq_decode_attention, ctypes.byref(cd), base, 8, 100, 0, base, None, base, 16, None) == WS
    assert call(L.tq_decode_attention, ctypes.byref(cd), base, 8, 100, 0, base, None, base + 8, ws_big, None) == WS
    assert call(L.tq_decode_attention_sparse, ctypes.byref(cd), base, 8, 100, 0, 1.5, base, None, base, ws_big,
                None) == ARG
    assert call(L.tq_decode_attention, ctypes.byref(cd), base, 8, 100, 0, base, None, base, ws_big, None) == HIP
    assert call(L.tq_decode_attention_append, ctypes.byref(cd), base, base, 99, base, 8, 100, 0, base, None, base,
                ws_big, None) == HIP
    assert call(L.tq_decode_attention_append, ctypes.byref(cd), None, base, 99, base, 8, 100, 0, base, None, base,
                ws_big, None) == ARG
    assert call(L.tq_decode_attention_append, ctypes.byref(cd), base, base, 1024, base, 8, 100, 0, base, None, base,
                ws_big, None) == CAP
    big = desc(d=256, kbits=4, vbits=5, cap=1 << 20, B=2, H=4)
    assert call(L.tq_decode_attention_noalloc, ctypes.byref(big), base, 64, 100000, 2000, base, None, None) == SCR
    assert call(L.tq_decode_workspace_init, None, 1 << 20, None) == ARG
    assert call(L.tq_decode_workspace_init, base, 1 << 10, None) == WS
    assert call(L.tq_decode_workspace_init, base, 1 << 20, None) == HIP
    for nbytes, sink in ((0, base), (16, None), (20, base), (32, base)):
        call(L.tq_read_probe, base, nbytes, sink, None)
    for bad in (None,):
        call(L.tq_quantize_append, bad, base, base, 1, 0, None)
        call(L.tq_decode_workspace_bytes, bad, 8, 1, 0)
        call(L.tq_dequantize, bad, 0, 0, 1, base, None)
    print(f"driven {n} calls")


if __name__ == "__main__":
    main(sys.argv[1])
