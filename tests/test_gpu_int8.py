"""GPU parity of the INT8 per-token absmax cache (mlxcel "TurboQuant KV
cache", "Available modes": int8) against the oracle: codes bit-exact against
the exact definition round(127 x / max|x|) and scales equal, dequantized rows, decode over
the GPU-written rows (both decode kernels: the matrix-core one takes INT8 on
both sides at head_dim 128, the plain split kernel every mix), paged
storage, and the policy's int8 mode."""
import os

import numpy as np
import pytest

import oracle
import synth
from parity import rows_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402
from compressed_decode_attention_append_amd import policy as P  # noqa: E402

S = tq.SideSpec


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


@pytest.fixture(params=["auto", "ref"])
def variant(request):
    old = os.environ.get("TQ_DECODE_VARIANT")
    os.environ["TQ_DECODE_VARIANT"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("TQ_DECODE_VARIANT", None)
    else:
        os.environ["TQ_DECODE_VARIANT"] = old


def _int8_rows(cache, side, lo, hi, logical=False):
    codes = (cache.logical if logical else cache.tensors.__getitem__)(side + "_codes")[:, :, lo:hi]
    norms = (cache.logical if logical else cache.tensors.__getitem__)(side + "_norms")[:, :, lo:hi]
    c = codes.cpu().numpy().view(np.int8)      # d bytes a row, coordinate j in byte j
    return c, norms.cpu().numpy()


def _rows(cache, side, length):
    spec = cache.k_spec if side == "k" else cache.v_spec
    if spec.mode == "fp16":
        return cache.tensors[side + "_fp16"][:, :, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        c, s = _int8_rows(cache, side, 0, length)
        return oracle.int8_dequantize(c, s)
    d = cache.head_dim
    R = oracle.rotation_matrix(cache.seed, d)
    cb, _ = oracle.lloyd_max(d, spec.bits)
    from parity import words_to_codes
    words = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy()
    norms = cache.tensors[side + "_norms"][:, :, :length].cpu().numpy().astype(np.float64)
    return oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, cb)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dist", ["iid", "channel"])
def test_int8_codes_and_scales(d, dist):
    B, H, cap = 2, 3, 300
    cache = tq.TQCache(B, H, d, cap, S("int8"), S("int8"))
    pos = 0
    for i, n in enumerate((130, 1, 17, 100)):
        k, v = synth.kv_numpy(50 + i, B, H, n, d, dist=dist, outlier_frac=0.01)
        cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), pos)
        torch.cuda.synchronize()
        for side, x in (("k", k), ("v", v)):
            c, s = _int8_rows(cache, side, pos, pos + n)
            c_o, s_o = oracle.int8_quantize(x)
            assert np.array_equal(c, c_o), f"{side}: {int(np.sum(c != c_o))} codes differ"
            assert np.array_equal(s, s_o), side
        pos += n
    # untouched rows stay zero
    assert int(cache.tensors["k_codes"][:, :, pos:].abs().sum()) == 0


def test_int8_codes_on_exact_half_steps():
    # rows whose elements sit exactly on half steps of the code grid (127 x /
    # max|x| = k + 1/2) or next to them: the encoder must round as the exact
    # definition does (ties to even), where dividing by the float32 scale
    # would not; 8192 rows through the encoder
    rng = np.random.default_rng(11)
    B, H, n, d = 1, 2, 4096, 128
    x = (rng.standard_normal((B, H, n, d)) * rng.uniform(0.01, 300.0, (B, H, n, 1))).astype(np.float16)
    x[:, :, :, 0] = np.float16(127.0)
    x[:, :, ::2, 1:40] = (rng.integers(-126, 126, (B, H, n // 2, 39)) + 0.5).astype(np.float16)
    x[:, :, 7, :8] = np.array([-34.6, 53.6, 39.16, 51.62, 23.88, -64.8, 92.9, -103.25], np.float16)
    cache = tq.TQCache(B, H, d, n, S("int8"), S("int8"))
    xt = torch.from_numpy(x).cuda()
    cache.quantize_append(xt, xt, 0)
    torch.cuda.synchronize()
    c, s = _int8_rows(cache, "k", 0, n)
    c_o, s_o = oracle.int8_quantize(x)
    assert np.array_equal(c, c_o), f"{int(np.sum(c != c_o))} codes differ"
    assert np.array_equal(s, s_o)


def test_int8_zero_rows_and_dequantize():
    B, H, d, cap = 1, 2, 128, 64
    k, v = synth.kv_numpy(60, B, H, 64, d)
    k[:, :, 5] = 0
    v[:, :, 9] = 0
    cache = tq.TQCache(B, H, d, cap, S("int8"), S("int8"))
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    for side, x in (("k", k), ("v", v)):
        out = cache.dequantize(side, 0, 64)
        torch.cuda.synchronize()
        c_o, s_o = oracle.int8_quantize(x)
        ref = oracle.int8_dequantize(c_o, s_o)
        got = out.cpu().numpy().astype(np.float64)
        assert np.allclose(got, ref, rtol=1e-7, atol=0), side
    c, s = _int8_rows(cache, "k", 5, 6)
    assert np.all(c == 0) and np.all(s == 0)


@pytest.mark.parametrize("kspec,vspec", [(S("int8"), S("int8")), (S("fp16"), S("int8")),
                                         (S("int8"), S("packed", 4)), (S("packed", 3), S("int8"))],
                         ids=["int8-int8", "fp16-int8", "int8-packed4", "packed3-int8"])
@pytest.mark.parametrize("length", [1, 65, 777])
def test_int8_decode(kspec, vspec, length, variant):
    B, H, Hq, d, cap = 2, 2, 8, 128, 800
    k, v = synth.kv_numpy(70, B, H, length, d, dist="channel", outlier_frac=0.01)
    cache = tq.TQCache(B, H, d, cap, kspec, vspec)
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    q = synth.q_numpy(71, B, Hq, d)
    out, sc = cache.decode_attention(torch.from_numpy(q).cuda(), length, scores=True)
    torch.cuda.synchronize()
    ref, s_ref = oracle.decode_attention(q, _rows(cache, "k", length), _rows(cache, "v", length))
    ok, worst = rows_close(sc.cpu().numpy(), s_ref)
    assert ok, f"scores: worst {worst}"
    ok, worst = rows_close(out.cpu().numpy(), ref)
    assert ok, f"out: worst {worst}"


@pytest.mark.parametrize("H,Hq,d", [(4, 4, 128), (1, 8, 128), (2, 16, 64), (1, 3, 256)],
                         ids=["g1_d128", "g8_d128", "g8_d64", "g3_d256"])
def test_int8_decode_group_sizes(H, Hq, d, variant):
    # query groups of one, three and eight heads per KV head: eight heads on
    # 64-position tiles take two softmax passes; d = 256 rows fall back to
    # 32-position tiles
    B, cap, length = 1, 700, 613
    k, v = synth.kv_numpy(72, B, H, length, d, dist="channel", outlier_frac=0.01)
    cache = tq.TQCache(B, H, d, cap, S("int8"), S("int8"))
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    q = synth.q_numpy(73, B, Hq, d)
    out, sc = cache.decode_attention(torch.from_numpy(q).cuda(), length, scores=True)
    torch.cuda.synchronize()
    ref, s_ref = oracle.decode_attention(q, _rows(cache, "k", length), _rows(cache, "v", length))
    ok, worst = rows_close(sc.cpu().numpy(), s_ref)
    assert ok, f"scores: worst {worst}"
    ok, worst = rows_close(out.cpu().numpy(), ref)
    assert ok, f"out: worst {worst}"


def test_int8_paged_matches_contiguous(variant):
    B, H, Hq, d, cap, bs = 2, 2, 8, 128, 512, 64
    k, v = synth.kv_numpy(80, B, H, 450, d)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(B * cap // bs).astype(np.int32).reshape(B, -1))
    a = tq.TQCache(B, H, d, cap, S("int8"), S("int8"))
    b = tq.TQCache(B, H, d, cap, S("int8"), S("int8"), block_table=perm, block_size=bs, num_blocks=B * cap // bs)
    for c in (a, b):
        c.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    q = torch.from_numpy(synth.q_numpy(81, B, Hq, d)).cuda()
    oa, ob = a.decode_attention(q, 450), b.decode_attention(q, 450)
    torch.cuda.synchronize()
    for name in a.tensors:
        assert torch.equal(a.tensors[name], b.logical(name)), name
    assert torch.equal(oa, ob)


def test_policy_int8_mode():
    B, H, Hq, d, cap = 1, 2, 4, 64, 200
    k, v = synth.kv_numpy(90, B, H, cap, d)
    dense = P.DenseKV(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 150)
    out = P.maybe_quantize([dense, dense], "int8", skip_last=True)
    assert isinstance(out[0], tq.TQCache) and out[0].k_spec.mode == "int8" and out[1] is dense
    torch.cuda.synchronize()
    c, s = _int8_rows(out[0], "v", 0, 150)
    c_o, s_o = oracle.int8_quantize(v[:, :, :150])
    assert np.array_equal(c, c_o) and np.array_equal(s, s_o)
