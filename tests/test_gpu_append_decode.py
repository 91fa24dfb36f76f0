"""The fused append-then-attend call (tq_decode_attention_append) against the
oracle and against the two separate calls it stands for.

Each case fills a cache with quantize_append, then writes one new position
per sequence at `offset` and attends over [0, length) in one call.  Checked:
* the rows written at `offset`: fp16 rows exactly; INT8 codes and scales
  equal the exact definition; packed codes equal the oracle's quantization
  of the new rows except within 1e-6 of a threshold, norms within 1e-6;
* scores and outputs against the oracle's attention over the rows the GPU
  wrote, within 2e-3 of each row's largest magnitude;
* the separate calls (tq_quantize_append, then tq_decode_attention) on a
  second cache filled the same way: outputs within the same tolerance, and
  bit-identical where the call makes those two calls itself (delegated
  sides, head_dim 64, an offset past the attended range, and any call that
  asks for scores).
"""
import numpy as np
import pytest

import oracle
import synth
from parity import codes_agree, rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

S = tq.SideSpec

# name, B, Hkv, Hq, d, capacity, filled, offset, length, K, V, block size (0: contiguous), splits, one launch
CASES = [
    ("asym_d128", 2, 2, 8, 128, 1400, 1336, 1336, 1337, S("fp16", 0), S("packed", 4), 0, 0, True),
    ("tq35_d128", 2, 2, 8, 128, 2100, 2099, 2099, 2100, S("packed", 3), S("packed", 4), 0, 0, True),
    ("tq35_splits3", 1, 2, 8, 128, 2100, 2099, 2099, 2100, S("packed", 3), S("packed", 4), 0, 3, True),
    ("k2v3_d128", 1, 4, 16, 128, 704, 699, 699, 700, S("packed", 2), S("packed", 3), 0, 0, True),
    ("g16_tq35", 1, 2, 32, 128, 900, 899, 899, 900, S("packed", 3), S("packed", 4), 0, 0, True),
    ("mid_offset", 1, 2, 8, 128, 1024, 1000, 517, 1000, S("packed", 3), S("packed", 4), 0, 2, True),
    ("asym_paged", 2, 2, 8, 128, 640, 600, 600, 601, S("fp16", 0), S("packed", 4), 64, 0, True),
    ("delegated", 1, 2, 16, 128, 960, 899, 899, 900, S("fp16", 0), S("delegated", 4, 64), 0, 0, False),
    ("int8", 1, 2, 8, 128, 704, 699, 699, 700, S("int8", 0), S("int8", 0), 0, 0, True),
    ("int8_g12_paged", 1, 2, 24, 128, 640, 600, 600, 601, S("int8", 0), S("int8", 0), 64, 0, True),
    ("d64", 1, 2, 4, 64, 300, 255, 255, 256, S("packed", 3), S("packed", 4), 0, 0, False),
    ("past_length", 1, 2, 8, 128, 800, 700, 750, 700, S("packed", 3), S("packed", 4), 0, 0, False),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


def _cache(case, seed):
    name, B, H, Hq, d, cap, filled, offset, length, ks, vs, bs, ns, fused = case
    kw = {}
    if bs:
        mb = cap // bs
        nb = B * mb + 1
        table = np.random.default_rng(seed).permutation(nb)[:B * mb].reshape(B, mb).astype(np.int32)
        kw = dict(block_table=torch.from_numpy(table), block_size=bs, num_blocks=nb)
    c = tq.TQCache(B, H, d, cap, ks, vs, device="cuda", **kw)
    for s0 in range(0, filled, 512):
        n = min(512, filled - s0)
        k, v = synth.kv_numpy(seed * 100 + s0, B, H, n, d, dist="channel", outlier_frac=0.01)
        c.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), s0)
    return c


def _view(cache, name):
    return cache.logical(name) if cache.paged else cache.tensors[name]


def _rows(cache, side, spec, length):
    d = cache.head_dim
    if spec.mode == "fp16":
        return _view(cache, side + "_fp16")[:, :, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        c = _view(cache, side + "_codes")[:, :, :length].cpu().numpy().view(np.int8)
        return oracle.int8_dequantize(c, _view(cache, side + "_norms")[:, :, :length].cpu().numpy())
    R = oracle.rotation_matrix(cache.seed, d)
    cb, _ = oracle.lloyd_max(d, spec.bits)
    words = _view(cache, side + "_codes")[:, :, :length].cpu().numpy()
    norms = _view(cache, side + "_norms")[:, :, :length].cpu().numpy().astype(np.float64)
    rows = oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, cb)
    if spec.mode == "delegated":
        n_cold = max(0, length - spec.hot)
        ring = cache.tensors[side + "_ring"].cpu().numpy()
        for t in range(n_cold, length):
            rows[:, :, t] = ring[:, :, t % spec.hot].astype(np.float64)
    return rows


def _check_row(cache, side, spec, x, offset):
    d = cache.head_dim
    if spec.mode == "fp16":
        got = _view(cache, side + "_fp16")[:, :, offset:offset + 1].cpu().numpy()
        assert np.array_equal(got, x), side
    elif spec.mode == "int8":
        c = _view(cache, side + "_codes")[:, :, offset:offset + 1].cpu().numpy().view(np.int8)
        s = _view(cache, side + "_norms")[:, :, offset:offset + 1].cpu().numpy()
        c_o, s_o = oracle.int8_quantize(x)
        assert np.array_equal(c, c_o) and np.array_equal(s, s_o), side
    elif spec.mode == "packed":
        R = oracle.rotation_matrix(cache.seed, d)
        _, t = oracle.lloyd_max(d, spec.bits)
        codes_o, n_o, y_o = oracle.quantize(x, R, t)
        words = _view(cache, side + "_codes")[:, :, offset:offset + 1].cpu().numpy()
        norms = _view(cache, side + "_norms")[:, :, offset:offset + 1].cpu().numpy()
        ok, ndiff, nnear = codes_agree(words_to_codes(words, spec.bits, d), codes_o, y_o, t)
        assert ok, f"{side}: {ndiff} codes differ outside the threshold band ({nnear} near)"
        assert np.all(np.abs(norms - n_o) <= 1e-6 * np.maximum(n_o, 1e-30)), side


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_decode(case):
    name, B, H, Hq, d, cap, filled, offset, length, ks, vs, bs, ns, fused = case
    print(f"{name}: B{B} Hkv{H} Hq{Hq} d{d} offset {offset} length {length} splits {ns}", flush=True)
    a = _cache(case, 11)
    b = _cache(case, 11)
    kn, vn = synth.kv_numpy(77, B, H, 1, d, dist="channel", outlier_frac=0.01)
    q = synth.q_numpy(78, B, Hq, d)
    kd, vd, qd = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(q).cuda()
    out = a.decode_attention_append(kd, vd, offset, qd, length, n_splits=ns)
    b.quantize_append(kd, vd, offset)
    out_b = b.decode_attention(qd, length, n_splits=ns)
    out_bs, sc_b = b.decode_attention(qd, length, n_splits=ns, scores=True)
    # asking for scores takes the two calls: bit-identical to them
    c = _cache(case, 11)
    out_c, sc_c = c.decode_attention_append(kd, vd, offset, qd, length, n_splits=ns, scores=True)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_bs) and torch.equal(sc_c, sc_b), "the call with scores must equal the separate calls"
    _check_row(a, "k", ks, kn, offset)
    if vs.mode != "delegated":
        _check_row(a, "v", vs, vn, offset)
    kr, vr = _rows(a, "k", ks, length), _rows(a, "v", vs, length)
    o_ref, s_ref = oracle.decode_attention(q, kr, vr)
    _, sc = a.decode_attention(qd, length, n_splits=ns, scores=True)  # the scores of the rows written
    ok, worst = rows_close(sc.cpu().numpy(), s_ref)
    assert ok, f"scores worst {worst}"
    ok, worst = rows_close(out.cpu().numpy(), o_ref)
    assert ok, f"out worst {worst}"
    if fused:
        ok, worst = rows_close(out.cpu().numpy(), out_b.cpu().numpy().astype(np.float64))
        assert ok, f"against the separate calls: worst {worst}"
    else:
        assert torch.equal(out, out_b), "the two-call path must equal the separate calls"


def test_append_decode_repeated_steps():
    # several decode steps in a row, each appending the next position and
    # attending over everything so far (the serving loop's pattern)
    B, H, Hq, d, cap = 2, 2, 8, 128, 700
    a = tq.TQCache(B, H, d, cap, S("packed", 3), S("packed", 4), device="cuda")
    k, v = synth.kv_numpy(5, B, H, 640, d, dist="channel", outlier_frac=0.01)
    a.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    ws = a.workspace(Hq, cap)
    for step in range(6):
        pos = 640 + step
        kn, vn = synth.kv_numpy(200 + step, B, H, 1, d, dist="channel", outlier_frac=0.01)
        q = synth.q_numpy(300 + step, B, Hq, d)
        out = a.decode_attention_append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), pos,
                                        torch.from_numpy(q).cuda(), pos + 1, workspace=ws)
        torch.cuda.synchronize()
        _check_row(a, "k", S("packed", 3), kn, pos)
        _check_row(a, "v", S("packed", 4), vn, pos)
        o_ref, _ = oracle.decode_attention(q, _rows(a, "k", S("packed", 3), pos + 1),
                                           _rows(a, "v", S("packed", 4), pos + 1))
        ok, worst = rows_close(out.cpu().numpy(), o_ref)
        assert ok, f"step {step}: out worst {worst}"
