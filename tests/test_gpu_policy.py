"""GPU checks of the host-side cache policy: the conversions it makes go
through tq_quantize_append and decode like any other cache (oracle parity on
the GPU-written codes), and conversion in chunks writes the same bits as one
append."""
import numpy as np
import pytest

import oracle
import synth
from parity import codes_agree, rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402
from compressed_decode_attention_append_amd import policy as P  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


def _dense(seed, B, H, cap, d, offset):
    k, v = synth.kv_numpy(seed, B, H, cap, d)
    k[:, :, offset:] = 0
    v[:, :, offset:] = 0
    return P.DenseKV(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), offset), k, v


def _rows(cache, side, length):
    spec = cache.k_spec if side == "k" else cache.v_spec
    if spec.mode == "fp16":
        return cache.tensors[side + "_fp16"][:, :, :length].cpu().numpy().astype(np.float64)
    d = cache.head_dim
    R = oracle.rotation_matrix(cache.seed, d)
    c, _ = oracle.lloyd_max(d, spec.bits)
    words = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy()
    norms = cache.tensors[side + "_norms"][:, :, :length].cpu().numpy().astype(np.float64)
    rows = oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, c)
    if spec.mode == "delegated":
        # the newest `hot` positions are fp16 in the ring, slot = position % hot
        ring = cache.tensors[side + "_ring"].cpu().numpy()
        for p in range(max(0, length - spec.hot), length):
            rows[:, :, p] = ring[:, :, p % spec.hot].astype(np.float64)
    return rows


def _check_codes(cache, side, x, length):
    spec = cache.k_spec if side == "k" else cache.v_spec
    d = cache.head_dim
    R = oracle.rotation_matrix(cache.seed, d)
    _, t = oracle.lloyd_max(d, spec.bits)
    codes_o, n_o, y_o = oracle.quantize(x[:, :, :length], R, t)
    words = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy()
    ok, ndiff, nnear = codes_agree(words_to_codes(words, spec.bits, d), codes_o, y_o, t)
    assert ok, f"{side}: {ndiff} codes differ outside the threshold band ({nnear} near)"
    norms = cache.tensors[side + "_norms"][:, :, :length].cpu().numpy()
    assert np.all(np.abs(norms - n_o) <= 1e-6 * np.maximum(n_o, 1e-30))


def _check_decode(cache, seed, q_heads, length):
    q = synth.q_numpy(seed, cache.batch, q_heads, cache.head_dim)
    out, sc = cache.decode_attention(torch.from_numpy(q).cuda(), length, scores=True)
    torch.cuda.synchronize()
    ref, s_ref = oracle.decode_attention(q, _rows(cache, "k", length), _rows(cache, "v", length))
    ok, worst = rows_close(sc.cpu().numpy(), s_ref)
    assert ok, f"scores: worst {worst}"
    ok, worst = rows_close(out.cpu().numpy(), ref)
    assert ok, f"out: worst {worst}"


def test_maybe_quantize_layers():
    B, H, Hq, d, cap = 1, 2, 4, 64, 320
    offsets = [0, 100, 300, 300]
    made = [_dense(11 + i, B, H, cap, d, off) for i, off in enumerate(offsets)]
    caches = [m[0] for m in made]
    out = P.maybe_quantize(caches, 3.5, quantized_kv_start=200)
    torch.cuda.synchronize()
    # empty dense cache -> empty TurboQuant cache of the same shape
    assert isinstance(out[0], tq.TQCache)
    assert (out[0].k_spec.bits, out[0].v_spec.bits) == (3, 4)
    assert out[0].capacity == cap and int(out[0].tensors["k_codes"].abs().sum()) == 0
    # shorter than quantized_kv_start: unchanged
    assert out[1] is caches[1]
    # converted: the oracle's codes, and a decode that matches the oracle
    c2 = out[2]
    assert isinstance(c2, tq.TQCache)
    _check_codes(c2, "k", made[2][1], 300)
    _check_codes(c2, "v", made[2][2], 300)
    _check_decode(c2, 5, Hq, 300)
    # the last layer stays full precision
    assert out[3] is caches[3]
    # a layer that is already TurboQuant is kept
    again = P.maybe_quantize(out, 3.5, quantized_kv_start=200)
    assert again[0] is out[0] and again[2] is out[2]


def test_from_dense_chunks_write_the_same_bits():
    B, H, d, cap = 2, 2, 128, 300
    dense, _, _ = _dense(23, B, H, cap, d, 290)
    k, v = P.mode_sides(3.5)
    a = P.from_dense(dense, k, v, chunk=64)
    b = P.from_dense(dense, k, v, chunk=4096)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        assert torch.equal(a.tensors[name], b.tensors[name]), name


@pytest.mark.parametrize("mode,boundary", [("turbo4", 1), ("turbo4-delegated", 0), ("fp16+turbo3", 0)])
def test_policy_layers_decode(mode, boundary):
    B, H, Hq, d, cap = 1, 2, 8, 128, 700
    sides = P.layer_sides(3, mode, skip_last=True, boundary_v=boundary, hot=64)
    sd = sides[0]
    assert sd is not None
    dense, k, v = _dense(31, B, H, cap, d, 650)
    cache = P.from_dense(dense, sd[0], sd[1], chunk=256)
    torch.cuda.synchronize()
    if sd[0].mode == "packed":
        _check_codes(cache, "k", k, 650)
    if sd[1].mode == "packed":
        _check_codes(cache, "v", v, 650)
    if sd[1].mode == "delegated":
        _check_codes(cache, "v", v, 650 - sd[1].hot)  # the cold rows
    _check_decode(cache, 7, Hq, 650)
