"""Paged (block-table) storage: the same kernels over block pools.

A paged cache and a contiguous one fed the same appends must hold the same
bits at every logical position, and decode must return bit-identical
scores and outputs (the split structure, and so every sum, is the same; the
pages report paged decode as byte-identical to the dense backend, mlxcel
"TurboQuant KV cache", "Paged cache and server batching").  The contiguous
path itself is checked against the oracle in test_gpu_parity.py; one case
here also checks the paged decode against the oracle directly."""
import os

import numpy as np
import pytest

import oracle
import synth
from parity import rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

S = tq.SideSpec

# name, B, Hkv, Hq, d, block_size, K, V
CASES = [
    ("tq35_d128", 2, 2, 8, 128, 64, S("packed", 3), S("packed", 4)),
    ("asym_d128", 2, 2, 8, 128, 32, S("fp16", 0), S("packed", 4)),
    ("sym4_d128", 1, 2, 8, 128, 128, S("packed", 4), S("packed", 4)),
    ("delegated_d128", 2, 2, 16, 128, 64, S("fp16", 0), S("delegated", 4, 64)),
    ("tq35_d64", 1, 2, 4, 64, 32, S("packed", 3), S("packed", 4)),
    ("fp16v_d128", 1, 2, 8, 128, 32, S("packed", 3), S("fp16", 0)),
    ("asym3_d128", 2, 2, 8, 128, 64, S("fp16", 0), S("packed", 3)),
    ("k3v3_d128", 1, 2, 8, 128, 32, S("packed", 3), S("packed", 3)),
    ("k2v3_d128", 2, 2, 8, 128, 32, S("packed", 2), S("packed", 3)),
    ("asym2_d128", 1, 2, 8, 128, 64, S("fp16", 0), S("packed", 2)),
    ("g16_tq35_d128", 1, 2, 32, 128, 64, S("packed", 3), S("packed", 4)),
]
CAP = 640
APPENDS = [(0, 300), (300, 1), (301, 216)]   # (offset, rows)
LENGTHS = [301, 517]


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


def _table(B, max_blocks, seed, spare=3):
    rng = np.random.default_rng(seed)
    n = B * max_blocks + spare
    ids = rng.permutation(n)[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    return torch.from_numpy(ids), n


def _pair(case, seed):
    name, B, H, Hq, d, bs, k, v = case
    contig = tq.TQCache(B, H, d, CAP, k, v, device="cuda")
    table, n = _table(B, CAP // bs, seed)
    paged = tq.TQCache(B, H, d, CAP, k, v, device="cuda", block_table=table, block_size=bs, num_blocks=n)
    for i, (off, rows) in enumerate(APPENDS):
        kx, vx = synth.kv_numpy(seed + i, B, H, rows, d, dist="channel", outlier_frac=0.01)
        kd, vd = torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda()
        contig.quantize_append(kd, vd, off)
        paged.quantize_append(kd, vd, off)
    torch.cuda.synchronize()
    return contig, paged


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_storage_and_decode_match_contiguous(case, dvariant):
    contig, paged = _pair(case, 1000 + CASES.index(case))
    for name in contig.tensors:
        a, b = contig.tensors[name], paged.logical(name)
        assert torch.equal(a, b), name
    Hq = case[3]
    # both through the same kernel; the delegated lengths start the hot
    # window off the 32-position grid (301 - 64, 517 - 64)
    for length in LENGTHS:
        q = torch.from_numpy(synth.q_numpy(77, case[1], Hq, case[4])).cuda()
        oc, sc = contig.decode_attention(q, length, scores=True)
        op, sp = paged.decode_attention(q, length, scores=True)
        torch.cuda.synchronize()
        assert torch.equal(sc, sp), f"scores differ at length {length}"
        assert torch.equal(oc, op), f"outputs differ at length {length}"


# appends whose offset and length are multiples of 16 take the matrix-core
# encoder's aligned paged path (one table entry per 16-row tile); the short
# and odd ones after them take the general path and the plain encoder
APPENDS_ALIGNED = [(0, 256), (256, 48), (304, 16), (320, 1), (321, 31)]


@pytest.mark.parametrize("case", [c for c in CASES if c[4] == 128], ids=[c[0] for c in CASES if c[4] == 128])
def test_paged_aligned_appends_match_contiguous(case):
    name, B, H, Hq, d, bs, k, v = case
    seed = 3000 + CASES.index(case)
    contig = tq.TQCache(B, H, d, CAP, k, v, device="cuda")
    table, n = _table(B, CAP // bs, seed)
    paged = tq.TQCache(B, H, d, CAP, k, v, device="cuda", block_table=table, block_size=bs, num_blocks=n)
    for i, (off, rows) in enumerate(APPENDS_ALIGNED):
        kx, vx = synth.kv_numpy(seed + i, B, H, rows, d, dist="channel", outlier_frac=0.01)
        kd, vd = torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda()
        contig.quantize_append(kd, vd, off)
        paged.quantize_append(kd, vd, off)
    torch.cuda.synchronize()
    for nm in contig.tensors:
        assert torch.equal(contig.tensors[nm], paged.logical(nm)), nm
    q = torch.from_numpy(synth.q_numpy(78, B, Hq, d)).cuda()
    # a delegated V is decoded at its appended length only (its ring holds
    # the newest positions appended)
    for length in ((352,) if v.mode == "delegated" else (320, 352)):
        oc, sc = contig.decode_attention(q, length, scores=True)
        op, sp = paged.decode_attention(q, length, scores=True)
        torch.cuda.synchronize()
        assert torch.equal(sc, sp) and torch.equal(oc, op), length


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_dequantize_matches_contiguous(case):
    contig, paged = _pair(case, 2000 + CASES.index(case))
    for side in ("k", "v"):
        if (case[6] if side == "k" else case[7]).mode == "fp16":
            continue
        for start, count in ((0, 517), (31, 65), (300, 1)):
            a = contig.dequantize(side, start, count)
            b = paged.dequantize(side, start, count)
            torch.cuda.synchronize()
            assert torch.equal(a, b), (side, start, count)


def test_shared_prefix_blocks():
    # two sequences whose first two blocks are the same pool blocks (a shared
    # prompt prefix stored once), then their own blocks
    B, H, Hq, d, bs = 2, 2, 8, 128, 64
    k, v = S("packed", 3), S("packed", 4)
    mb = CAP // bs
    table = np.zeros((B, mb), np.int32)
    table[:, :2] = [5, 9]
    table[0, 2:] = np.arange(10, 10 + mb - 2)
    table[1, 2:] = np.arange(30, 30 + mb - 2)
    paged = tq.TQCache(B, H, d, CAP, k, v, device="cuda", block_table=torch.from_numpy(table), block_size=bs,
                       num_blocks=64)
    contig = tq.TQCache(B, H, d, CAP, k, v, device="cuda")
    kx, vx = synth.kv_numpy(41, 1, H, 2 * bs, d)
    kx, vx = np.repeat(kx, B, axis=0), np.repeat(vx, B, axis=0)       # the shared prefix
    ky, vy = synth.kv_numpy(42, B, H, 100, d)                         # each sequence's own
    for c in (contig, paged):
        c.quantize_append(torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda(), 0)
        c.quantize_append(torch.from_numpy(ky).cuda(), torch.from_numpy(vy).cuda(), 2 * bs)
    torch.cuda.synchronize()
    for name in contig.tensors:
        assert torch.equal(contig.tensors[name], paged.logical(name)), name
    q = torch.from_numpy(synth.q_numpy(43, B, Hq, d)).cuda()
    length = 2 * bs + 100
    oc = contig.decode_attention(q, length)
    op = paged.decode_attention(q, length)
    torch.cuda.synchronize()
    assert torch.equal(oc, op)
    # and against the oracle, over the rows the paged cache holds
    R = oracle.rotation_matrix(0, d)
    rows = {}
    for side, bits in (("k", 3), ("v", 4)):
        c, _ = oracle.lloyd_max(d, bits)
        words = paged.logical(side + "_codes")[:, :, :length].cpu().numpy()
        norms = paged.logical(side + "_norms")[:, :, :length].cpu().numpy().astype(np.float64)
        rows[side] = oracle.dequantize(words_to_codes(words, bits, d), norms, R, c)
    ref, _ = oracle.decode_attention(q.cpu().numpy(), rows["k"], rows["v"])
    ok, worst = rows_close(op.cpu().numpy(), ref)
    assert ok, f"out: worst {worst}"


@pytest.mark.parametrize("variant", ["auto", "ref"])
@pytest.mark.parametrize("ns", [2, 3, 7])
@pytest.mark.parametrize("case", [CASES[4], ("tq35_d128_bs32", 2, 2, 8, 128, 32, S("packed", 3), S("packed", 4)),
                                  ("asym_d128_bs64", 2, 3, 15, 128, 64, S("fp16", 0), S("packed", 4))],
                         ids=["tq35_d64", "tq35_d128_bs32", "asym_d128_bs64"])
def test_paged_split_counts_match_contiguous(case, ns, variant, monkeypatch):
    # explicit split counts: the plain kernel's split lengths are off the
    # 32-position grid, so its tiles cross block boundaries (32-position
    # tiles at d = 64, 64-position tiles over 32-position blocks at d = 128);
    # the matrix-core kernel rounds its split lengths up to that grid, since
    # each of its 32-position chunks must lie in one block (length 574 over
    # 2 splits once started a split at 287, and those chunks read across
    # block boundaries)
    monkeypatch.setenv("TQ_DECODE_VARIANT", variant)
    contig, paged = _pair(case, 2024 + ns)
    for length in LENGTHS + [574]:
        q = torch.from_numpy(synth.q_numpy(78, case[1], case[3], case[4])).cuda()
        oc, sc = contig.decode_attention(q, length, n_splits=ns, scores=True)
        op, sp = paged.decode_attention(q, length, n_splits=ns, scores=True)
        torch.cuda.synchronize()
        assert torch.equal(sc, sp), f"scores differ at length {length}"
        assert torch.equal(oc, op), f"outputs differ at length {length}"
