"""Host-side tests of the C ABI (no GPU needed): every symbol the header
declares is exported, the host helpers agree with the oracle, and every
error path is taken before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_decode_attention_append_amd as tq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tq_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 9
    L = tq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_missing_library_raises_tq_error(monkeypatch):
    # the product path fails loudly (a TQError naming the missing library)
    # when libtq.so is absent, and never falls back to anything else
    monkeypatch.setattr(tq, "_lib", None)
    monkeypatch.setattr(tq, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libtq.so"))
    with pytest.raises(tq.TQError, match="not built"):
        tq.lib()
    assert tq.status_string(-1) == "libtq not built"


def test_status_strings():
    for s in range(0, -9, -1):
        assert tq.status_string(s) not in ("", "unknown status")
    assert tq.status_string(-99) == "unknown status"


def test_split_bits_and_row_words():
    assert tq.split_bits(3.5) == oracle.split_bits(3.5) == (3, 4)
    assert tq.split_bits(4.2) == (4, 5)
    assert tq.split_bits(8) == (8, 8)
    for bad in (0.5, 8.5, 9, float("nan")):
        with pytest.raises(tq.TQError):
            tq.split_bits(bad)
    for d in (32, 64, 128, 256):
        for b in range(1, 9):
            assert tq.row_words(d, b) == oracle.row_words(d, b)
    with pytest.raises(tq.TQError):
        tq.row_words(80, 4)
    with pytest.raises(tq.TQError):
        tq.row_words(128, 9)


@pytest.mark.parametrize("seed", [0, 1, 12345, 2**63 + 17])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_sign_words_match_oracle(seed, d):
    w = tq.sign_words(seed, d)
    bits = np.array([(int(w[j // 32]) >> (j % 32)) & 1 for j in range(d)])
    want = (oracle.sign_vector(seed, d) < 0).astype(int)
    assert np.array_equal(bits, want)


@pytest.mark.parametrize("d", [32, 64, 128, 256, 1024])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_codebook_builder_matches_oracle(d, bits):
    c, t = tq.build_codebook(d, bits)
    co, to = oracle.lloyd_max(d, bits)
    tol = 2e-12 if (d <= 256 and bits <= 4) else 1e-10
    assert np.max(np.abs(c - co)) <= tol * max(1.0, np.max(np.abs(co)) * 0 + 1.0)
    assert np.max(np.abs(t - to)) <= tol
    assert t[(1 << bits) // 2 - 1] == 0.0
    assert np.array_equal(c, -c[::-1])
    # the fp32 copies the kernels use agree to within one fp32 ulp
    assert np.all(np.abs(c.astype(np.float32) - co.astype(np.float32)) <= np.spacing(np.abs(co).astype(np.float32)))


def test_codebook_builder_six_bits():
    c, t = tq.build_codebook(128, 6)
    co, to = oracle.lloyd_max(128, 6)
    assert np.max(np.abs(c - co)) <= 1e-10


def test_codebook_builder_rejects():
    with pytest.raises(tq.TQError):
        tq.build_codebook(128, 0)
    with pytest.raises(tq.TQError):
        tq.build_codebook(96, 3)


# ---- error paths: nothing is launched ------------------------------------

class _Fake:
    """Host buffers standing in for device pointers; never dereferenced on
    the error paths exercised here."""

    def __init__(self):
        self.buf = np.zeros(1 << 16, np.uint8)
        self.c = np.zeros(256, np.float32)

    def p(self, off=0):
        return self.buf.ctypes.data + off


def _desc(f, d=128, kmode=1, vmode=1, kb=3, vb=4, hot=256, cap=1024, B=2, H=4):
    c = tq.tq_cache()
    c.batch, c.kv_heads, c.head_dim, c.capacity, c.seed = B, H, d, cap, 0
    for side, mode, bits in ((c.k, kmode, kb), (c.v, vmode, vb)):
        side.mode, side.bits, side.hot = mode, bits, hot
        side.centroids = f.c.ctypes.data
        side.thresholds = f.c.ctypes.data
        side.codes, side.norms, side.fp16 = f.p(0), f.p(256), f.p(512)
    return c


def _qa(c, f, n=4, off=0):
    return tq.lib().tq_quantize_append(ctypes.byref(c), f.p(1024), f.p(2048), n, off, None)


def _dec(c, f, Hq=8, length=100, ns=0, ws_bytes=1 << 30, ws_off=0, q=True, out=True):
    return tq.lib().tq_decode_attention(ctypes.byref(c), f.p(4096) if q else None, Hq, length, ns,
                                        f.p(8192) if out else None, None, f.p(ws_off) if ws_bytes else None,
                                        ws_bytes, None)


def test_quantize_append_errors():
    f = _Fake()
    assert _qa(_desc(f, d=96), f) == tq.TQ_ERR_HEAD_DIM
    assert _qa(_desc(f, d=512), f) == tq.TQ_ERR_HEAD_DIM
    assert _qa(_desc(f, kb=0), f) == tq.TQ_ERR_BITS
    assert _qa(_desc(f, vb=9), f) == tq.TQ_ERR_BITS
    assert _qa(_desc(f, kmode=2), f) == tq.TQ_ERR_MODE   # delegated K
    assert _qa(_desc(f, vmode=7), f) == tq.TQ_ERR_MODE
    assert _qa(_desc(f, vmode=2, hot=0), f) == tq.TQ_ERR_ARG
    assert _qa(_desc(f), f, n=-1) == tq.TQ_ERR_ARG
    assert _qa(_desc(f, cap=10), f, n=8, off=3) == tq.TQ_ERR_CAPACITY
    assert _qa(_desc(f), f, n=1, off=-1) == tq.TQ_ERR_CAPACITY
    c = _desc(f)
    c.k.codes = None
    assert _qa(c, f) == tq.TQ_ERR_ARG
    c = _desc(f, kmode=0)
    c.k.fp16 = None
    assert _qa(c, f) == tq.TQ_ERR_ARG
    c = _desc(f)
    c.v.centroids = None
    assert _qa(c, f) == tq.TQ_ERR_ARG
    c = _desc(f)
    c.batch = 0
    assert _qa(c, f) == tq.TQ_ERR_ARG
    assert tq.lib().tq_quantize_append(None, f.p(), f.p(), 1, 0, None) == tq.TQ_ERR_ARG
    assert tq.lib().tq_quantize_append(ctypes.byref(_desc(f)), None, f.p(), 1, 0, None) == tq.TQ_ERR_ARG
    # n_new = 0 is a no-op, even with null rows
    assert tq.lib().tq_quantize_append(ctypes.byref(_desc(f)), None, None, 0, 0, None) == tq.TQ_OK


def test_decode_errors():
    f = _Fake()
    c = _desc(f)
    assert _dec(c, f, Hq=6) == tq.TQ_ERR_ARG          # not a multiple of Hkv
    assert _dec(c, f, Hq=2) == tq.TQ_ERR_ARG          # fewer than Hkv
    assert _dec(c, f, length=2000) == tq.TQ_ERR_CAPACITY
    assert _dec(c, f, length=-1) == tq.TQ_ERR_CAPACITY
    assert _dec(c, f, ns=-1) == tq.TQ_ERR_ARG
    assert _dec(c, f, q=False) == tq.TQ_ERR_ARG
    assert _dec(c, f, out=False) == tq.TQ_ERR_ARG
    need = tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 100, 0)
    assert need > 0
    assert _dec(c, f, ws_bytes=need - 1) == tq.TQ_ERR_WORKSPACE
    assert _dec(c, f, ws_bytes=0) == tq.TQ_ERR_WORKSPACE
    assert tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 6, 100, 0) == 0
    assert tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 5000, 0) == 0
    assert _dec(_desc(f, d=100), f) == tq.TQ_ERR_HEAD_DIM


def test_append_decode_errors():
    # the fused append-then-attend call checks every argument of both steps
    # before anything is launched (no GPU is touched on these paths)
    f = _Fake()
    c = _desc(f)
    need = tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 100, 0)

    def call(k=True, v=True, offset=99, q=True, Hq=8, length=100, ns=0, out=True, ws_bytes=need, cache=c):
        return tq.lib().tq_decode_attention_append(ctypes.byref(cache), f.p(1024) if k else None,
                                                   f.p(2048) if v else None, offset, f.p(4096) if q else None,
                                                   Hq, length, ns, f.p(8192) if out else None, None,
                                                   f.p(0) if ws_bytes else None, ws_bytes, None)
    assert call(k=False) == tq.TQ_ERR_ARG
    assert call(v=False) == tq.TQ_ERR_ARG
    assert call(q=False) == tq.TQ_ERR_ARG
    assert call(out=False) == tq.TQ_ERR_ARG
    assert call(offset=-1) == tq.TQ_ERR_CAPACITY
    assert call(offset=1024) == tq.TQ_ERR_CAPACITY      # capacity 1024
    assert call(Hq=6) == tq.TQ_ERR_ARG
    assert call(length=1025) == tq.TQ_ERR_CAPACITY
    assert call(ns=-1) == tq.TQ_ERR_ARG
    assert call(ws_bytes=need - 1) == tq.TQ_ERR_WORKSPACE
    assert call(cache=_desc(f, d=100)) == tq.TQ_ERR_HEAD_DIM
    assert call(cache=_desc(f, kb=0)) == tq.TQ_ERR_BITS


def test_decode_workspace_grows_with_splits():
    f = _Fake()
    c = _desc(f)
    a = tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 1000, 1)
    b = tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 1000, 4)
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0


def test_dequantize_errors():
    f = _Fake()
    L = tq.lib()
    assert L.tq_dequantize(ctypes.byref(_desc(f)), 2, 0, 1, f.p(), None) == tq.TQ_ERR_ARG
    assert L.tq_dequantize(ctypes.byref(_desc(f, kmode=0)), 0, 0, 1, f.p(), None) == tq.TQ_ERR_MODE
    assert L.tq_dequantize(ctypes.byref(_desc(f, cap=10)), 1, 5, 6, f.p(), None) == tq.TQ_ERR_CAPACITY
    assert L.tq_dequantize(ctypes.byref(_desc(f)), 1, 0, 1, None, None) == tq.TQ_ERR_ARG
    assert L.tq_dequantize(ctypes.byref(_desc(f)), 1, 0, 0, None, None) == tq.TQ_OK


def test_read_probe_argument_errors():
    # every rejection happens before a launch, so no GPU is needed
    L = tq.lib()
    fake = ctypes.c_void_p(4096)  # never dereferenced: rejected first
    assert L.tq_read_probe(fake, 16, None, None) == tq.TQ_ERR_ARG             # no sink
    assert L.tq_read_probe(None, 16, fake, None) == tq.TQ_ERR_ARG             # no buffer
    assert L.tq_read_probe(fake, 20, fake, None) == tq.TQ_ERR_ARG             # not a multiple of 16
    assert L.tq_read_probe(ctypes.c_void_p(4100), 32, fake, None) == tq.TQ_ERR_ARG  # misaligned


def test_paged_descriptor_errors():
    # paged storage: block_size a multiple of 32, max_blocks >= 1, num_blocks
    # >= 1 and capacity == max_blocks * block_size; checked before any launch
    f = _Fake()
    table = np.zeros(64, np.int32)

    def paged(bs, mb, cap, nb=16):
        c = _desc(f, cap=cap)
        c.block_table, c.block_size, c.max_blocks, c.num_blocks = table.ctypes.data, bs, mb, nb
        return c

    for bs, mb, cap, nb in ((48, 4, 192, 16), (16, 8, 128, 16), (0, 4, 0, 16), (64, 0, 0, 16), (64, 4, 192, 16),
                            (64, 4, 320, 16), (64, 4, 256, 0), (64, 4, 256, -3)):
        c = paged(bs, mb, cap, nb)
        assert _qa(c, f, n=0) == tq.TQ_ERR_ARG, (bs, mb, cap)
        assert tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 0, 0) == 0
        assert tq.lib().tq_dequantize(ctypes.byref(c), 1, 0, 0, None, None) == tq.TQ_ERR_ARG
    ok = paged(64, 4, 256)
    assert _qa(ok, f, n=0) == tq.TQ_OK
    assert tq.lib().tq_decode_workspace_bytes(ctypes.byref(ok), 8, 256, 0) > 0
    assert _qa(ok, f, n=4, off=253) == tq.TQ_ERR_CAPACITY


def test_noalloc_decode_errors():
    # the allocation-free decode validates like tq_decode_attention and
    # refuses a call whose workspace would exceed its fixed scratch, all
    # before any launch or device set-up
    f = _Fake()
    L = tq.lib()

    def na(c, Hq=8, length=100, ns=0, q=True, out=True):
        return L.tq_decode_attention_noalloc(ctypes.byref(c), f.p(4096) if q else None, Hq, length, ns,
                                             f.p(8192) if out else None, None, None)

    assert na(_desc(f, d=96)) == tq.TQ_ERR_HEAD_DIM
    assert na(_desc(f), q=False) == tq.TQ_ERR_ARG
    assert na(_desc(f), out=False) == tq.TQ_ERR_ARG
    assert na(_desc(f), Hq=6) == tq.TQ_ERR_ARG
    assert na(_desc(f), ns=-1) == tq.TQ_ERR_ARG
    assert na(_desc(f), length=2000) == tq.TQ_ERR_CAPACITY
    # the plain kernel's partials at 2000 splits of 64 query heads, d = 256:
    # far beyond 16 MiB
    big = _desc(f, d=256, kb=4, vb=5, cap=1 << 20, B=2, H=4)
    assert L.tq_decode_workspace_bytes(ctypes.byref(big), 64, 100000, 2000) > tq.TQ_NOALLOC_SCRATCH_BYTES
    assert na(big, Hq=64, length=100000, ns=2000) == tq.TQ_ERR_SCRATCH
    assert "16 MiB" in tq.status_string(tq.TQ_ERR_SCRATCH)


def test_workspace_init_errors():
    # the counter-region set-up: a null, short or misaligned workspace is
    # refused before any launch
    L = tq.lib()
    fake = np.zeros(1 << 20, np.uint8)
    base = (fake.ctypes.data + 255) & ~255
    assert tq.WORKSPACE_COUNTER_BYTES == 256 * 1024
    assert L.tq_decode_workspace_init(None, 1 << 20, None) == tq.TQ_ERR_ARG
    assert L.tq_decode_workspace_init(ctypes.c_void_p(base), 256 * 1024 - 16, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_decode_workspace_init(ctypes.c_void_p(base + 16), 1 << 19, None) == tq.TQ_ERR_WORKSPACE


def test_workspace_bytes_cover_the_counters():
    f = _Fake()
    for kmode, vmode, d, Hq in ((1, 1, 128, 8), (0, 1, 128, 8), (1, 1, 64, 4), (3, 3, 128, 8)):
        c = _desc(f, kmode=kmode, vmode=vmode, d=d)
        for length in (0, 1, 1000):
            assert tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), Hq, length, 0) >= tq.WORKSPACE_COUNTER_BYTES


def test_cache_checks_its_block_table_on_the_host():
    # the binding holds the table when it builds the descriptor, so it
    # refuses entries outside [0, num_blocks) there (the library guards them
    # on the device)
    torch = pytest.importorskip("torch")
    S = tq.SideSpec
    good = torch.arange(8, dtype=torch.int32).reshape(2, 4)
    c = tq.TQCache(2, 2, 64, 256, S("packed", 3), S("packed", 4), device="cpu", block_table=good, block_size=64,
                   num_blocks=8)
    assert c.desc.num_blocks == 8 and c.desc.max_blocks == 4 and c.desc.block_size == 64
    for bad, nb in ((torch.tensor([[0, 1, 2, 3], [4, 5, 6, 8]], dtype=torch.int32), 8),
                    (torch.tensor([[0, 1, 2, 3], [4, 5, -1, 7]], dtype=torch.int32), 8),
                    (good, 0)):
        with pytest.raises(ValueError):
            tq.TQCache(2, 2, 64, 256, S("packed", 3), S("packed", 4), device="cpu", block_table=bad, block_size=64,
                       num_blocks=nb)


def test_sparse_v_threshold_errors():
    # the threshold must lie in [0, 1); checked before any launch
    f = _Fake()
    c = _desc(f)
    for tau in (-0.1, 1.0, 2.0, float("nan")):
        r = tq.lib().tq_decode_attention_sparse(ctypes.byref(c), f.p(4096), 8, 100, 0, tau, f.p(8192), None,
                                                f.p(0), 1 << 30, None)
        assert r == tq.TQ_ERR_ARG, tau


def test_int8_side_arguments():
    # an INT8 side needs its codes and scales; its bit field is not read
    f = _Fake()
    c = _desc(f, kmode=3, vmode=3, kb=0, vb=77)
    assert _qa(c, f, n=0) == tq.TQ_OK
    assert tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), 8, 100, 0) > 0
    c.k.codes = None
    assert _qa(c, f, n=0) == tq.TQ_ERR_ARG
    c = _desc(f, kmode=0, vmode=3)
    c.v.norms = None
    assert _qa(c, f, n=0) == tq.TQ_ERR_ARG
    # delegated stays V-only; INT8 K with a delegated V is fine
    assert _qa(_desc(f, kmode=3, vmode=2), f, n=0) == tq.TQ_OK


def test_decode_workspace_head_groups():
    # the matrix-core kernel runs a query group of G > 8 heads as ceil(G / 8)
    # head groups, each with partials for 8 heads per split; an explicit
    # split count gives splits of a multiple of 32 positions
    f = _Fake()
    for Hkv, Hq, ns, splits in ((2, 96, 1, 1), (2, 96, 5, 5), (1, 12, 7, 7), (1, 8, 3, 3), (2, 4, 300, 32)):
        c = _desc(f, d=128, B=1, H=Hkv, kb=3, vb=4)
        got = tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), Hq, 1000, ns)
        G = Hq // Hkv
        groups, per = (G + 7) // 8, min(G, 8)
        want = 65536 * 4 + (Hkv * groups * splits * per * 132 * 4 + 255) // 256 * 256
        assert got == want, (Hkv, Hq, ns, got, want)


def test_decode_workspace_any_group_size():
    # the plain kernel takes any query group (eight heads a block, more
    # blocks per KV head beyond that) and any split count: the workspace is
    # the partials' size, counters first
    f = _Fake()
    for d, Hkv, Hq in ((256, 1, 256), (128, 2, 96), (32, 1, 3)):
        # (5-bit sides: the matrix-core kernel takes 2 to 4 bits at d = 128)
        c = _desc(f, d=d, B=1, H=Hkv, kb=5, vb=5)
        for ns in (0, 1, 5, 300):
            got = tq.lib().tq_decode_workspace_bytes(ctypes.byref(c), Hq, 1000, ns)
            assert got > 0, (d, Hq, ns)
            if ns:
                # max/sum plus two d-wide accumulators per (query head, split),
                # each region 256-byte aligned, after 256 KiB of counters
                units = Hq * ns
                want = 65536 * 4
                for n in (units * 2, units * d, units * d):
                    want += (n * 4 + 255) // 256 * 256
                assert got == want, (d, Hq, ns, got, want)
