"""Sparse-V decode (tq_decode_attention_sparse) against the exact decode and
the oracle's bound on what dropping small-weight values may change.

Inputs are peaked on purpose: the first 64 positions of each KV head point
along the queries' direction, so every later chunk's weights are far below
the threshold and its values are skipped; the oracle bound is computed on
the GPU-written cache rows."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from parity import rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

S = tq.SideSpec
CASES = [
    ("tq35", S("packed", 3), S("packed", 4)),
    ("asym", S("fp16", 0), S("packed", 4)),
    ("delegated", S("fp16", 0), S("delegated", 4, 128)),
    ("int8", S("int8", 0), S("int8", 0)),
    ("asym3", S("fp16", 0), S("packed", 3)),
    ("k2v3", S("packed", 2), S("packed", 3)),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


@pytest.fixture(params=["auto", "ref"])
def dvariant(request):
    old = os.environ.get("TQ_DECODE_VARIANT")
    os.environ["TQ_DECODE_VARIANT"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("TQ_DECODE_VARIANT", None)
    else:
        os.environ["TQ_DECODE_VARIANT"] = old


def _peaked(B, H, Hq, d, T, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, H, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    k = rng.standard_normal((B, H, T, d))
    k[:, :, :64] = 8.0 * u[:, :, None, :] + 0.5 * rng.standard_normal((B, H, 64, d))
    v = rng.standard_normal((B, H, T, d))
    G = Hq // H
    q = 32.0 * np.repeat(u, G, axis=1) + 0.1 * rng.standard_normal((B, Hq, d))
    return k.astype(np.float16), v.astype(np.float16), q.astype(np.float16)


def _rows(cache, side, length):
    spec = cache.k_spec if side == "k" else cache.v_spec
    if spec.mode == "fp16":
        return cache.tensors[side + "_fp16"][:, :, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        codes = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy().view(np.int8)  # byte j = coordinate j
        return oracle.int8_dequantize(codes, cache.tensors[side + "_norms"][:, :, :length].cpu().numpy())
    d = cache.head_dim
    R = oracle.rotation_matrix(cache.seed, d)
    c, _ = oracle.lloyd_max(d, spec.bits)
    words = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy()
    norms = cache.tensors[side + "_norms"][:, :, :length].cpu().numpy().astype(np.float64)
    rows = oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, c)
    if spec.mode == "delegated":
        ring = cache.tensors[side + "_ring"].cpu().numpy()
        for p in range(max(0, length - spec.hot), length):
            rows[:, :, p] = ring[:, :, p % spec.hot].astype(np.float64)
    return rows


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("tau", [1e-3, 0.2])
def test_sparse_v_within_bound(case, tau, dvariant):
    name, ks, vs = case
    B, H, Hq, d, T = 1, 2, 8, 128, 1000
    k, v, q = _peaked(B, H, Hq, d, T, 7)
    cache = tq.TQCache(B, H, d, 1024, ks, vs)
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qd = torch.from_numpy(q).cuda()
    exact = cache.decode_attention(qd, T)
    sparse = cache.decode_attention(qd, T, sparse_v=tau)
    torch.cuda.synchronize()
    exact, sparse = exact.cpu().numpy().astype(np.float64), sparse.cpu().numpy().astype(np.float64)
    kr, vr = _rows(cache, "k", T), _rows(cache, "v", T)
    bound = oracle.sparse_v_bound(q, kr, vr, tau)
    scale = np.max(np.abs(exact), axis=-1, keepdims=True)
    # what the skipped values may change, plus the kernels' own rounding
    assert np.all(np.abs(sparse - exact) <= bound * (1 + 1e-3) + 1e-5 * scale)
    # values were skipped (the later chunks' weights are ~e^-20 of the peak)
    assert not np.array_equal(sparse, exact)
    # and the sparse output is within tolerance of the exact attention
    ref, _ = oracle.decode_attention(q, kr, vr)
    ok, worst = rows_close(sparse, ref, rel=2e-3 + float(np.max(bound / scale)))
    assert ok, f"worst {worst}"


def test_zero_threshold_is_the_exact_call():
    B, H, Hq, d, T = 2, 2, 8, 128, 700
    k, v, q = _peaked(B, H, Hq, d, T, 9)
    cache = tq.TQCache(B, H, d, 1024, S("packed", 3), S("packed", 4))
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qd = torch.from_numpy(q).cuda()
    exact = cache.decode_attention(qd, T)
    ws = cache.workspace(Hq, T)
    out = torch.empty_like(exact)
    r = tq.lib().tq_decode_attention_sparse(ctypes.byref(cache.desc), qd.data_ptr(), Hq, T, 0, 0.0,
                                            out.data_ptr(), None, ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    assert r == tq.TQ_OK
    assert torch.equal(out, exact)


def _periodic(B, H, Hq, d, T, period, seed):
    """Heavy hitters at the first two positions of every ``period``: the
    chunks between them are skippable and the chunk holding the next pair
    is not, so a decode that predicts a skip from the chunk before must
    still fetch that chunk's values."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, H, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    k = rng.standard_normal((B, H, T, d))
    hot = (np.arange(T) % period) < 2
    k[:, :, hot] = 8.0 * u[:, :, None, :] + 0.5 * rng.standard_normal((B, H, int(hot.sum()), d))
    v = rng.standard_normal((B, H, T, d))
    G = Hq // H
    q = 32.0 * np.repeat(u, G, axis=1) + 0.1 * rng.standard_normal((B, Hq, d))
    return k.astype(np.float16), v.astype(np.float16), q.astype(np.float16)


@pytest.mark.parametrize("case", CASES[:2], ids=[c[0] for c in CASES[:2]])
@pytest.mark.parametrize("period", [96, 384])
def test_sparse_v_periodic_peaks(case, period, dvariant):
    name, ks, vs = case
    B, H, Hq, d, T = 2, 2, 8, 128, 5000
    k, v, q = _periodic(B, H, Hq, d, T, period, 11)
    cache = tq.TQCache(B, H, d, T, ks, vs)
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qd = torch.from_numpy(q).cuda()
    tau = 1e-3
    exact = cache.decode_attention(qd, T)
    sparse = cache.decode_attention(qd, T, sparse_v=tau)
    torch.cuda.synchronize()
    exact, sparse = exact.cpu().numpy().astype(np.float64), sparse.cpu().numpy().astype(np.float64)
    kr, vr = _rows(cache, "k", T), _rows(cache, "v", T)
    bound = oracle.sparse_v_bound(q, kr, vr, tau)
    scale = np.max(np.abs(exact), axis=-1, keepdims=True)
    assert np.all(np.abs(sparse - exact) <= bound * (1 + 1e-3) + 1e-5 * scale)
    assert not np.array_equal(sparse, exact)
    # the heavy hitters' values dominate: dropping any of them would move the
    # output by far more than the bound
    ref, _ = oracle.decode_attention(q, kr, vr)
    ok, worst = rows_close(sparse, ref, rel=2e-3 + float(np.max(bound / scale)))
    assert ok, f"worst {worst}"


@pytest.mark.parametrize("case", CASES[:2] + CASES[3:], ids=[c[0] for c in CASES[:2] + CASES[3:]])
def test_sparse_v_paged_within_bound(case, dvariant):
    # the skips and the reload of a predicted-skippable chunk's values go
    # through the block table (blocks in a shuffled order): the paged sparse
    # decode stays within the oracle bound of the exact attention, and skips
    name, ks, vs = case
    B, H, Hq, d, T, bs = 2, 2, 8, 128, 3000, 64
    cap = 3008
    k, v, q = _periodic(B, H, Hq, d, T, 160, 13)
    nb = B * cap // bs
    table = torch.from_numpy(np.random.default_rng(5).permutation(nb).astype(np.int32).reshape(B, cap // bs))
    paged = tq.TQCache(B, H, d, cap, ks, vs, block_table=table, block_size=bs, num_blocks=nb)
    paged.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qd = torch.from_numpy(q).cuda()
    tau = 1e-3
    exact = paged.decode_attention(qd, T)
    sparse = paged.decode_attention(qd, T, sparse_v=tau)
    torch.cuda.synchronize()
    exact, sparse = exact.cpu().numpy().astype(np.float64), sparse.cpu().numpy().astype(np.float64)
    logical = {}
    for side in ("k", "v"):
        spec = ks if side == "k" else vs
        if spec.mode == "fp16":
            logical[side] = paged.logical(side + "_fp16")[:, :, :T].cpu().numpy().astype(np.float64)
        elif spec.mode == "int8":
            codes = paged.logical(side + "_codes")[:, :, :T].cpu().numpy().view(np.int8)
            logical[side] = oracle.int8_dequantize(codes, paged.logical(side + "_norms")[:, :, :T].cpu().numpy())
        else:
            R = oracle.rotation_matrix(paged.seed, d)
            c, _ = oracle.lloyd_max(d, spec.bits)
            words = paged.logical(side + "_codes")[:, :, :T].cpu().numpy()
            norms = paged.logical(side + "_norms")[:, :, :T].cpu().numpy().astype(np.float64)
            logical[side] = oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, c)
    bound = oracle.sparse_v_bound(q, logical["k"], logical["v"], tau)
    scale = np.max(np.abs(exact), axis=-1, keepdims=True)
    assert np.all(np.abs(sparse - exact) <= bound * (1 + 1e-3) + 1e-5 * scale)
    assert not np.array_equal(sparse, exact)


@pytest.mark.parametrize("case", CASES[:2] + CASES[3:], ids=[c[0] for c in CASES[:2] + CASES[3:]])
def test_sparse_v_deterministic_and_layout_independent(case, dvariant):
    # which chunks are skipped depends only on the data and the fixed chunk
    # order: repeated calls give the same bits, and a paged cache (shuffled
    # blocks) gives the bits of a contiguous one
    name, ks, vs = case
    B, H, Hq, d, T, bs = 2, 2, 8, 128, 3000, 64
    cap = 3008
    k, v, q = _periodic(B, H, Hq, d, T, 160, 17)
    nb = B * cap // bs
    table = torch.from_numpy(np.random.default_rng(6).permutation(nb).astype(np.int32).reshape(B, cap // bs))
    contig = tq.TQCache(B, H, d, cap, ks, vs)
    paged = tq.TQCache(B, H, d, cap, ks, vs, block_table=table, block_size=bs, num_blocks=nb)
    for c in (contig, paged):
        c.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qd = torch.from_numpy(q).cuda()
    runs = [contig.decode_attention(qd, T, sparse_v=1e-3, scores=True) for _ in range(5)]
    op, sp_ = paged.decode_attention(qd, T, sparse_v=1e-3, scores=True)
    torch.cuda.synchronize()
    for o, sc in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(sc, runs[0][1])
    assert torch.equal(op, runs[0][0]) and torch.equal(sp_, runs[0][1])


@pytest.mark.parametrize("Hq", [6, 16], ids=["g3", "g8"])
def test_sparse_v_group_sizes(Hq, dvariant):
    # groups of three (padding heads in the four-head layout) and eight query
    # heads per KV head: the skip test and the block maxima cover the real
    # heads only
    B, H, d, T = 1, 2, 128, 4000
    k, v, q = _periodic(B, H, Hq, d, T, 256, 19)
    cache = tq.TQCache(B, H, d, T, S("packed", 3), S("packed", 4))
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qd = torch.from_numpy(q).cuda()
    tau = 1e-3
    exact = cache.decode_attention(qd, T)
    sparse = cache.decode_attention(qd, T, sparse_v=tau)
    torch.cuda.synchronize()
    exact, sparse = exact.cpu().numpy().astype(np.float64), sparse.cpu().numpy().astype(np.float64)
    kr, vr = _rows(cache, "k", T), _rows(cache, "v", T)
    bound = oracle.sparse_v_bound(q, kr, vr, tau)
    scale = np.max(np.abs(exact), axis=-1, keepdims=True)
    assert np.all(np.abs(sparse - exact) <= bound * (1 + 1e-3) + 1e-5 * scale)
    assert not np.array_equal(sparse, exact)
