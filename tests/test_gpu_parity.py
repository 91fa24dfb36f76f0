"""GPU parity of libtq against the CPU oracle, element by element, on seeded
synthetic inputs at sizes the oracle finishes in seconds (several tiles and a
ragged tail).  Every call goes through the C ABI."""
import math
import os
import zlib

import numpy as np
import pytest

import oracle
import synth
from parity import codes_agree, rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check_packed(cache, side, x, pos, seed=0, bits=None):
    """GPU-written rows [pos, pos + n) of a packed side versus the oracle's
    quantization of the same fp16 rows."""
    d = cache.head_dim
    bits = bits or (cache.k_spec.bits if side == "k" else cache.v_spec.bits)
    R = oracle.rotation_matrix(seed, d)
    _, t = oracle.lloyd_max(d, bits)
    codes_o, n_o, y_o = oracle.quantize(x, R, t)
    n = x.shape[2]
    words = cache.tensors[side + "_codes"][:, :, pos:pos + n].cpu().numpy()
    norms = cache.tensors[side + "_norms"][:, :, pos:pos + n].cpu().numpy()
    got = words_to_codes(words, bits, d)
    ok, ndiff, nnear = codes_agree(got, codes_o, y_o, t)
    assert ok, f"{side}: {ndiff} codes differ outside the threshold band ({nnear} near)"
    # packed words are exactly the oracle's packing of the GPU codes
    assert np.array_equal(oracle.pack_codes(got, bits), words.view(np.uint32))
    assert np.all(np.abs(norms - n_o) <= 1e-6 * np.maximum(n_o, 1e-30))
    return got, norms


def _oracle_rows(cache, side, length):
    """float64 rows [0, length) of one side as the decode must see them,
    rebuilt by the oracle from what the GPU wrote."""
    spec = cache.k_spec if side == "k" else cache.v_spec
    d = cache.head_dim
    if spec.mode == "fp16":
        return cache.tensors[side + "_fp16"][:, :, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        codes = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy().view(np.int8)  # byte j = coordinate j
        return oracle.int8_dequantize(codes, cache.tensors[side + "_norms"][:, :, :length].cpu().numpy())
    R = oracle.rotation_matrix(cache.seed, d)
    c, _ = oracle.lloyd_max(d, spec.bits)

    def packed(lo, hi):
        words = cache.tensors[side + "_codes"][:, :, lo:hi].cpu().numpy()
        norms = cache.tensors[side + "_norms"][:, :, lo:hi].cpu().numpy().astype(np.float64)
        return oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, c)

    if spec.mode == "packed":
        return packed(0, length)
    hot = spec.hot
    out = np.zeros((cache.batch, cache.kv_heads, length, d))
    n_cold = max(0, length - hot)
    if n_cold:
        out[:, :, :n_cold] = packed(0, n_cold)
    ring = cache.tensors[side + "_ring"].cpu().numpy()
    for p in range(n_cold, length):
        out[:, :, p] = ring[:, :, p % hot].astype(np.float64)
    return out


@pytest.fixture(params=["auto", "plain"])
def qvariant(request):
    """Runs a test with the library's own choice of quantize kernel (the
    matrix-core encoder where it applies) and again with the plain kernel
    forced (TQ_QUANTIZE_VARIANT=plain)."""
    old = os.environ.get("TQ_QUANTIZE_VARIANT")
    os.environ["TQ_QUANTIZE_VARIANT"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("TQ_QUANTIZE_VARIANT", None)
    else:
        os.environ["TQ_QUANTIZE_VARIANT"] = old


@pytest.mark.parametrize("d,kb,vb,B,H,n,off", [
    (64, 3, 4, 1, 2, 256, 0),      # the 3.5-bit d=64 workload, whole
    (128, 3, 4, 2, 3, 301, 7),     # ragged count at an offset
    (128, 4, 4, 1, 2, 190, 0),
    (128, 1, 2, 2, 3, 40, 3),      # 1- and 2-bit words from several lanes
    (128, 3, 4, 1, 1, 16, 0),      # exactly one tile
    (128, 4, 3, 3, 2, 17, 5),      # every tile crosses a (batch, head) boundary
    (128, 2, 1, 1, 1, 15, 0),      # too short for the matrix-core encoder
    (32, 1, 2, 2, 2, 77, 5),
    (256, 5, 8, 1, 2, 65, 3),
    (128, 6, 7, 1, 1, 33, 0),
])
def test_quantize_append_packed(d, kb, vb, B, H, n, off, qvariant):
    k, v = synth.kv_numpy(100 + d + n, B, H, n, d, dist="channel", outlier_frac=0.01)
    cache = tq.TQCache(B, H, d, off + n + 9, tq.SideSpec("packed", kb), tq.SideSpec("packed", vb))
    cache.quantize_append(_dev(k), _dev(v), off)
    torch.cuda.synchronize()
    _check_packed(cache, "k", k, off)
    _check_packed(cache, "v", v, off)
    for side in ("k", "v"):
        untouched = torch.cat([cache.tensors[side + "_codes"][:, :, :off], cache.tensors[side + "_codes"][:, :, off + n:]], 2)
        assert int(untouched.abs().sum()) == 0


def test_quantize_zero_and_tiny_rows(qvariant):
    d = 128
    k = np.zeros((1, 1, 20, d), np.float16)  # 20 rows: the matrix-core encoder takes them
    k[0, 0, 1, 5] = np.float16(6e-8)        # smallest subnormal
    k[0, 0, 2, :] = np.float16(65504.0)     # largest finite
    k[0, 0, 3, ::3] = np.float16(-1.0)
    k[0, 0, 4:] = synth.kv_numpy(3, 1, 1, 16, d)[0][0, 0]
    cache = tq.TQCache(1, 1, d, 20, tq.SideSpec("packed", 3), tq.SideSpec("packed", 4))
    cache.quantize_append(_dev(k), _dev(k), 0)
    torch.cuda.synchronize()
    _check_packed(cache, "k", k, 0)
    _check_packed(cache, "v", k, 0)
    codes = words_to_codes(cache.tensors["k_codes"][0, 0, 0:1].cpu().numpy(), 3, d)
    assert np.all(codes == 3)   # zero row: every code L/2 - 1
    assert float(cache.tensors["k_norms"][0, 0, 0]) == 0.0


def test_quantize_append_fp16_side(qvariant):
    d, B, H, n = 128, 2, 2, 50
    k, v = synth.kv_numpy(7, B, H, n, d)
    cache = tq.TQCache(B, H, d, 64, tq.SideSpec("fp16"), tq.SideSpec("packed", 4))
    cache.quantize_append(_dev(k), _dev(v), 10)
    torch.cuda.synchronize()
    assert np.array_equal(cache.tensors["k_fp16"][:, :, 10:60].cpu().numpy(), k)
    assert int(cache.tensors["k_fp16"][:, :, :10].abs().sum()) == 0
    _check_packed(cache, "v", v, 10)


@pytest.mark.parametrize("kb,vb", [(3, 4), (4, 4), (1, 2)])
def test_quantize_kernels_agree(kb, vb):
    """The matrix-core encoder and the plain kernel write the same words and
    norms, up to the threshold band, on the 32K-context distribution."""
    d, B, H, n = 128, 2, 4, 1000
    k, v = synth.kv_numpy(77 + kb, B, H, n, d, dist="channel", outlier_frac=0.01)
    out = {}
    for var in ("auto", "plain"):
        os.environ["TQ_QUANTIZE_VARIANT"] = var
        cache = tq.TQCache(B, H, d, n, tq.SideSpec("packed", kb), tq.SideSpec("packed", vb))
        cache.quantize_append(_dev(k), _dev(v), 0)
        torch.cuda.synchronize()
        out[var] = {key: cache.tensors[key].cpu().numpy() for key in ("k_codes", "k_norms", "v_codes", "v_norms")}
    os.environ.pop("TQ_QUANTIZE_VARIANT", None)
    R = oracle.rotation_matrix(0, d)
    for side, bits, x in (("k", kb, k), ("v", vb, v)):
        _, t = oracle.lloyd_max(d, bits)
        _, _, y = oracle.quantize(x, R, t)
        a = words_to_codes(out["auto"][side + "_codes"], bits, d)
        b = words_to_codes(out["plain"][side + "_codes"], bits, d)
        ok, ndiff, _ = codes_agree(a, b, y, t)
        assert ok, f"{side}: {ndiff} codes differ outside the band"
        na, nb = out["auto"][side + "_norms"], out["plain"][side + "_norms"]
        assert np.all(np.abs(na - nb) <= 1e-6 * np.abs(nb) + 1e-30)


@pytest.mark.parametrize("chunks,hot", [
    ([300], 64), ([1] * 70 + [200], 64), ([100, 100, 100], 64), ([63, 1, 1, 130, 5], 64),
    ([700], 256), ([256, 1, 256], 256),
])
def test_delegated_append(chunks, hot):
    d, B, H = 128, 2, 2
    T = sum(chunks)
    k, v = synth.kv_numpy(31 + T, B, H, T, d, dist="channel")
    cache = tq.TQCache(B, H, d, T, tq.SideSpec("fp16"), tq.SideSpec("delegated", 4, hot))
    ref = oracle.DelegatedSide(B, H, T, d, 4, seed=0, hot=hot)
    off = 0
    for n in chunks:
        cache.quantize_append(_dev(k[:, :, off:off + n]), _dev(v[:, :, off:off + n]), off)
        ref.append(v[:, :, off:off + n], off)
        off += n
    torch.cuda.synchronize()
    assert np.array_equal(cache.tensors["v_ring"].cpu().numpy(), ref.ring)
    n_cold = max(0, T - hot)
    _, t = oracle.lloyd_max(d, 4)
    got = words_to_codes(cache.tensors["v_codes"][:, :, :n_cold].cpu().numpy(), 4, d)
    _, _, y = oracle.quantize(v[:, :, :n_cold], ref.cold.R, t)
    ok, ndiff, _ = codes_agree(got, ref.cold.codes[:, :, :n_cold], y, t)
    assert ok, ndiff
    norms = cache.tensors["v_norms"][:, :, :n_cold].cpu().numpy()
    assert np.all(np.abs(norms - ref.cold.norms[:, :, :n_cold]) <= 1e-6 * np.abs(ref.cold.norms[:, :, :n_cold]) + 1e-30)
    assert int(cache.tensors["v_codes"][:, :, n_cold:].abs().sum()) == 0


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4), (256, 2)])
def test_dequantize(d, bits):
    B, H, n = 1, 2, 129
    k, v = synth.kv_numpy(5, B, H, n, d, dist="channel", outlier_frac=0.01)
    cache = tq.TQCache(B, H, d, n, tq.SideSpec("packed", bits), tq.SideSpec("packed", bits))
    cache.quantize_append(_dev(k), _dev(v), 0)
    got = cache.dequantize("v", 3, 100).cpu().numpy()
    ref = _oracle_rows(cache, "v", n)[:, :, 3:103]
    ok, worst = rows_close(got, ref, 1e-5)
    assert ok, worst


DECODE_CASES = [
    # name, B, Hkv, Hq, d, T, k side, v side, dist
    ("tq35_d64", 1, 2, 4, 64, 256, ("packed", 3), ("packed", 4), "iid"),
    ("sym4_d128", 1, 8, 32, 128, 1500, ("packed", 4), ("packed", 4), "channel"),
    ("asym_d128", 2, 2, 8, 128, 1337, ("fp16", 0), ("packed", 4), "channel"),
    ("tq35_d128", 2, 2, 8, 128, 2100, ("packed", 3), ("packed", 4), "channel"),
    ("delegated", 2, 2, 16, 128, 900, ("fp16", 0), ("delegated", 4), "channel"),
    ("delegated_short", 1, 2, 16, 128, 200, ("fp16", 0), ("delegated", 4), "channel"),
    ("fp16_fp16", 1, 2, 4, 64, 333, ("fp16", 0), ("fp16", 0), "iid"),
    ("d32_mqa", 1, 1, 8, 32, 97, ("packed", 2), ("packed", 5), "iid"),
    ("d256", 1, 2, 4, 256, 130, ("packed", 4), ("packed", 3), "iid"),
    # query-group sizes of the plain kernel's head blocks: one head, three
    # (arrays sized for four), twelve (two blocks of six); fp16 rows at
    # d = 256 (more row pieces than the lanes' prefetch slots)
    ("mha_d128", 2, 4, 4, 128, 300, ("packed", 3), ("packed", 4), "channel"),
    ("g3_d64", 1, 2, 6, 64, 250, ("fp16", 0), ("packed", 2), "iid"),
    ("g12_d128", 1, 1, 12, 128, 200, ("packed", 4), ("packed", 4), "iid"),
    ("fp16_d256", 1, 1, 2, 256, 150, ("fp16", 0), ("fp16", 0), "iid"),
    # 96 query heads on one KV head: twelve head blocks of eight
    ("g96_d128", 1, 1, 96, 128, 150, ("packed", 2), ("packed", 2), "iid"),
    # the i.i.d. reading of the 3.5-bit and asymmetric workloads' "same K/V
    # distribution as config 1" (the most diffuse softmax) on the matrix-core
    # kernel's shapes
    ("tq35_d128_iid", 2, 2, 8, 128, 2100, ("packed", 3), ("packed", 4), "iid"),
    ("asym_d128_iid", 2, 2, 8, 128, 1337, ("fp16", 0), ("packed", 4), "iid"),
    ("sym4_d128_iid", 1, 8, 32, 128, 1500, ("packed", 4), ("packed", 4), "iid"),
    # INT8 on both sides (the matrix-core kernel's original-domain mode):
    # groups of one, four and eight heads, both readings
    ("int8_d128", 2, 2, 8, 128, 1900, ("int8", 0), ("int8", 0), "channel"),
    ("int8_d128_iid", 1, 8, 32, 128, 1500, ("int8", 0), ("int8", 0), "iid"),
    ("int8_mha", 2, 4, 4, 128, 300, ("int8", 0), ("int8", 0), "channel"),
    ("int8_g8", 1, 1, 8, 128, 613, ("int8", 0), ("int8", 0), "iid"),
    # query groups that leave padding columns in the matrix-core kernel's
    # head layouts (three of four, five of eight)
    ("int8_g3", 1, 2, 6, 128, 700, ("int8", 0), ("int8", 0), "iid"),
    ("int8_g5", 1, 1, 5, 128, 500, ("int8", 0), ("int8", 0), "channel"),
    # 3-bit V on the matrix-core kernel: fp16 K (the turbo3-asym mode), 3-bit
    # K (3.0 bits), 4-bit K beside it (K tables of their own), a delegated
    # 3-bit cold tail, eight and five heads a group
    ("asym3_d128", 2, 2, 8, 128, 1337, ("fp16", 0), ("packed", 3), "channel"),
    ("asym3_d128_iid", 1, 8, 32, 128, 1500, ("fp16", 0), ("packed", 3), "iid"),
    ("k3v3_d128", 2, 2, 8, 128, 2100, ("packed", 3), ("packed", 3), "iid"),
    ("k4v3_d128", 1, 2, 16, 128, 900, ("packed", 4), ("packed", 3), "channel"),
    ("delegated3", 2, 2, 16, 128, 900, ("fp16", 0), ("delegated", 3), "channel"),
    ("k3v3_g5", 1, 1, 5, 128, 500, ("packed", 3), ("packed", 3), "channel"),
    # 2-bit codes on the matrix-core kernel: 2.5 bits (2-bit K, 3-bit V),
    # 2.0 bits, fp16 K beside 2-bit V, a delegated 2-bit cold tail, three
    # heads a group
    ("k2v3_d128", 2, 2, 8, 128, 1337, ("packed", 2), ("packed", 3), "iid"),
    ("k2v2_d128", 1, 8, 32, 128, 1500, ("packed", 2), ("packed", 2), "channel"),
    ("asym2_d128", 1, 2, 16, 128, 900, ("fp16", 0), ("packed", 2), "iid"),
    ("delegated2", 1, 2, 8, 128, 700, ("fp16", 0), ("delegated", 2), "channel"),
    ("k2v2_g3", 1, 2, 6, 128, 613, ("packed", 2), ("packed", 2), "iid"),
    # query groups above 8 heads on the matrix-core kernel (head groups of
    # 8, the last one smaller for 12, 20 and 24)
    ("g16_tq35", 2, 2, 32, 128, 1500, ("packed", 3), ("packed", 4), "channel"),
    ("g16_asym_iid", 1, 4, 64, 128, 1337, ("fp16", 0), ("packed", 4), "iid"),
    ("g20_delegated", 1, 2, 40, 128, 700, ("fp16", 0), ("delegated", 4), "channel"),
    ("g12_int8", 1, 2, 24, 128, 613, ("int8", 0), ("int8", 0), "iid"),
]


def _build(case, extra=0, seed=0):
    name, B, Hkv, Hq, d, T, ks, vs, dist = case
    k, v = synth.kv_numpy(zlib.crc32(name.encode()) % 1000 + seed, B, Hkv, T, d, dist=dist,
                          outlier_frac=0.01 if dist == "channel" else 0.0)
    q = synth.q_numpy(zlib.crc32(name.encode()) % 1000 + seed, B, Hq, d)
    kspec = tq.SideSpec(ks[0], ks[1])
    vspec = tq.SideSpec(vs[0], vs[1], 256 if name == "delegated_short" else 128)
    cache = tq.TQCache(B, Hkv, d, T + extra, kspec, vspec, seed=seed)
    cache.quantize_append(_dev(k), _dev(v), 0)
    return cache, k, v, q


@pytest.fixture(params=["auto", "ref"])
def variant(request):
    """Runs a test with the library's own choice of decode kernel and again
    with the plain split kernel forced (TQ_DECODE_VARIANT=ref)."""
    old = os.environ.get("TQ_DECODE_VARIANT")
    os.environ["TQ_DECODE_VARIANT"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("TQ_DECODE_VARIANT", None)
    else:
        os.environ["TQ_DECODE_VARIANT"] = old


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_attention(case, variant):
    cache, k, v, q = _build(case, extra=5)
    T = k.shape[2]
    out, sc = cache.decode_attention(_dev(q), T, scores=True)
    torch.cuda.synchronize()
    kr = _oracle_rows(cache, "k", T)
    vr = _oracle_rows(cache, "v", T)
    o_ref, s_ref = oracle.decode_attention(q, kr, vr)
    ok, worst = rows_close(sc.cpu().numpy(), s_ref)
    print(f"{case[0]} {variant}: scores worst rel {worst:.3e}")
    assert ok, f"scores: worst {worst}"
    ok, worst = rows_close(out.cpu().numpy(), o_ref)
    print(f"{case[0]} {variant}: out worst rel {worst:.3e}")
    assert ok, f"out: worst {worst}"


SPLIT_CASES = DECODE_CASES[1:5] + [c for c in DECODE_CASES if c[0] in ("int8_d128", "asym3_d128", "k3v3_d128", "k2v3_d128", "g16_tq35")]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_decode_split_counts_agree(case, variant):
    cache, k, v, q = _build(case)
    T = k.shape[2]
    outs = [cache.decode_attention(_dev(q), T, n_splits=ns).cpu().numpy() for ns in (1, 3, 7, 16)]
    for o in outs[1:]:
        ok, worst = rows_close(o, outs[0], 1e-5)
        assert ok, worst


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_decode_variants_agree(case):
    cache, k, v, q = _build(case)
    T = k.shape[2]
    outs = {}
    for var in ("auto", "ref"):
        os.environ["TQ_DECODE_VARIANT"] = var
        outs[var] = cache.decode_attention(_dev(q), T).cpu().numpy()
    os.environ.pop("TQ_DECODE_VARIANT", None)
    ok, worst = rows_close(outs["auto"], outs["ref"], 1e-3)
    assert ok, worst


def test_decode_workspace_reuse_across_shapes():
    """The counter region left zero by one call serves the next call, even
    when the next call has a different shape or split count."""
    case = DECODE_CASES[3]
    cache, k, v, q = _build(case)
    T = k.shape[2]
    plan = ((3, T), (16, T), (0, 700), (0, T))
    need = max(cache.workspace_bytes(q.shape[1], length, ns) for ns, length in plan + ((16, T),))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ref = cache.decode_attention(_dev(q), T, n_splits=16, workspace=ws).cpu().numpy()
    for ns, length in plan:
        out = cache.decode_attention(_dev(q), length, n_splits=ns, workspace=ws).cpu().numpy()
        if length == T:
            ok, worst = rows_close(out, ref, 1e-5)
            assert ok, (ns, worst)
    assert int(ws[: 65536 * 4].view(torch.int32).abs().sum()) == 0


def test_decode_prefix_lengths(variant):
    case = DECODE_CASES[3]
    cache, k, v, q = _build(case)
    for length in (1, 2, 63, 64, 65, 1000):
        out = cache.decode_attention(_dev(q), length).cpu().numpy()
        kr = _oracle_rows(cache, "k", length)
        vr = _oracle_rows(cache, "v", length)
        o_ref, _ = oracle.decode_attention(q, kr, vr)
        ok, worst = rows_close(out, o_ref)
        assert ok, (length, worst)
    out = cache.decode_attention(_dev(q), 0).cpu().numpy()
    assert np.all(out == 0)


def test_decode_deterministic(variant):
    cache, k, v, q = _build(DECODE_CASES[3])
    T = k.shape[2]
    a = cache.decode_attention(_dev(q), T).cpu().numpy()
    b = cache.decode_attention(_dev(q), T).cpu().numpy()
    assert np.array_equal(a, b)


def test_quantize_deterministic():
    d, B, H, n = 128, 2, 2, 300
    k, v = synth.kv_numpy(9, B, H, n, d, dist="channel")
    words = []
    for _ in range(2):
        cache = tq.TQCache(B, H, d, n, tq.SideSpec("packed", 3), tq.SideSpec("packed", 4))
        cache.quantize_append(_dev(k), _dev(v), 0)
        words.append((cache.tensors["k_codes"].cpu().numpy(), cache.tensors["v_norms"].cpu().numpy()))
    assert np.array_equal(words[0][0], words[1][0]) and np.array_equal(words[0][1], words[1][1])


def test_end_to_end_against_oracle_quantization():
    """Oracle quantize -> oracle decode versus GPU quantize -> GPU decode."""
    case = DECODE_CASES[0]
    cache, k, v, q = _build(case)
    T = k.shape[2]
    out = cache.decode_attention(_dev(q), T).cpu().numpy()
    d = k.shape[-1]
    ks = oracle.PackedSide(1, 2, T, d, 3, 0)
    vs = oracle.PackedSide(1, 2, T, d, 4, 0)
    ks.write(k, 0)
    vs.write(v, 0)
    o_ref, _ = oracle.decode_attention(q, ks.rows(0, T), vs.rows(0, T))
    ok, worst = rows_close(out, o_ref)
    assert ok, worst


@pytest.mark.parametrize("nbytes", [0, 16, 48, 4096 * 16 + 48, 3 * 1024 * 1024 + 16 * 37])
def test_read_probe_xor(nbytes):
    # the probe's sink is the xor of every 32-bit word it streamed
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    words = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = words.to("cuda:0")
    sink = torch.full((1,), 12345, dtype=torch.int32, device="cuda:0")
    tq.read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words.numpy().view(np.uint32)) if nbytes else np.uint32(0)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
