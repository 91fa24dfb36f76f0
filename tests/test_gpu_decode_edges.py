"""Decode parity on edge-case rows, through both decode kernels, against the
oracle's float64 attention over the rows it rebuilds from what the GPU wrote:

* zero rows (norm 0: the codes of the middle cell, dequantized to 0) in K,
  in V and in both, mixed with ordinary rows;
* rows of fp16's largest magnitude (65504);
* row norms spanning nine decades (1e-4 .. 1e5) inside every 32-position
  chunk, for K and V independently and with one factor per position, so a
  head's weight can fall on rows whose value norm is far below the largest
  one seen;
* large logits (a peaked softmax);
* the same rows in INT8 caches (both sides), and with 3- and 2-bit codes
  (3-bit V beside fp16 K and beside 3-bit K; 2-bit K beside 2- and 3-bit V).

The tolerance is the parity tests' own: per row, ||x - ref||_inf <= 2e-3
||ref||_inf, for the scaled logits and for the outputs.
"""
import os
import zlib

import numpy as np
import pytest

import oracle
import synth
from parity import rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402


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


def _rows(cache, side, length):
    spec = cache.k_spec if side == "k" else cache.v_spec
    d = cache.head_dim
    if spec.mode == "fp16":
        return cache.tensors[side + "_fp16"][:, :, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        codes = cache.tensors[side + "_codes"][:, :, :length].cpu().numpy().view(np.int8)  # byte j = coordinate j
        return oracle.int8_dequantize(codes, cache.tensors[side + "_norms"][:, :, :length].cpu().numpy())
    R = oracle.rotation_matrix(cache.seed, d)
    c, _ = oracle.lloyd_max(d, spec.bits)
    n_cold = length if spec.mode == "packed" else max(0, length - spec.hot)
    out = np.zeros((cache.batch, cache.kv_heads, length, d))
    if n_cold:
        words = cache.tensors[side + "_codes"][:, :, :n_cold].cpu().numpy()
        norms = cache.tensors[side + "_norms"][:, :, :n_cold].cpu().numpy().astype(np.float64)
        out[:, :, :n_cold] = oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, c)
    if spec.mode == "delegated":
        ring = cache.tensors[side + "_ring"].cpu().numpy()
        for p in range(n_cold, length):
            out[:, :, p] = ring[:, :, p % spec.hot].astype(np.float64)
    return out


def _decade_factors(rng, shape, lo=-4.0, hi=5.0, d=128):
    """Per-position factors that give N(0, 1) rows of d coordinates norms
    10^u, u uniform in [lo, hi], so every 32-position chunk spans the range."""
    u = rng.uniform(lo, hi, shape)
    return (10.0 ** u / np.sqrt(d)).astype(np.float64)


def _case(name):
    """(k, v, q, k side, v side) of one edge case: B 2, 2 KV heads, 8 query
    heads, head_dim 128, 777 positions (several splits and a ragged tail)."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    B, H, Hq, T, d = 2, 2, 8, 777, 128
    k, v = synth.kv_numpy(len(name), B, H, T, d, dist="channel", outlier_frac=0.01)
    q = synth.q_numpy(len(name) + 1, B, Hq, d).astype(np.float64)
    k, v = k.astype(np.float64), v.astype(np.float64)
    ks, vs = ("packed", 3), ("packed", 4)
    if name.startswith("zero_rows"):
        k[:, :, ::5] = 0.0
        v[:, :, ::5] = 0.0
        k[:, :, 1::7] = 0.0
        v[:, :, 2::11] = 0.0
        k[:, :, 700:] = 0.0            # a run of zero keys through the tail
    elif name.startswith("fp16_max"):
        sgn = np.where(rng.random((B, H, T, d)) < 0.5, -1.0, 1.0)
        v[:, :, 3::9] = 65504.0 * sgn[:, :, 3::9]
        k[:, :, 5::13] = 65504.0 * sgn[:, :, 5::13]
        q = q / 4096.0                 # logits of the largest keys stay O(100)
    elif name.startswith("norm_decades_shared"):
        f = _decade_factors(rng, (B, H, T, 1))
        k = rng.standard_normal((B, H, T, d)) * f
        v = rng.standard_normal((B, H, T, d)) * f
        q = q * 3e-3                   # largest logits about +-30
    elif name.startswith("norm_decades"):
        k = rng.standard_normal((B, H, T, d)) * _decade_factors(rng, (B, H, T, 1))
        v = rng.standard_normal((B, H, T, d)) * _decade_factors(rng, (B, H, T, 1))
        q = q * 3e-3
    elif name.startswith("large_logits"):
        q = q * 24.0                   # logits of several hundred
    if name.endswith("_asym"):
        ks = ("fp16", 0)
    if name.endswith("_delegated"):
        ks, vs = ("fp16", 0), ("delegated", 4)
    if name.endswith("_int8"):
        ks, vs = ("int8", 0), ("int8", 0)
    if name.endswith("_asym3"):
        ks, vs = ("fp16", 0), ("packed", 3)
    if name.endswith("_k3v3"):
        ks, vs = ("packed", 3), ("packed", 3)
    if name.endswith("_k2v2"):
        ks, vs = ("packed", 2), ("packed", 2)
    if name.endswith("_k2v3"):
        ks, vs = ("packed", 2), ("packed", 3)
    return k.astype(np.float16), v.astype(np.float16), q.astype(np.float16), ks, vs


CASES = ["zero_rows", "zero_rows_asym", "fp16_max", "fp16_max_asym", "norm_decades", "norm_decades_asym",
         "norm_decades_delegated", "norm_decades_shared", "large_logits", "large_logits_asym",
         "zero_rows_int8", "fp16_max_int8", "norm_decades_int8", "large_logits_int8",
         "zero_rows_k3v3", "fp16_max_asym3", "norm_decades_asym3", "large_logits_k3v3",
         "zero_rows_k2v2", "fp16_max_k2v3", "norm_decades_k2v2", "large_logits_k2v3"]


@pytest.mark.parametrize("name", CASES)
def test_decode_edge_rows(name, variant):
    k, v, q, ks, vs = _case(name)
    B, H, T, d = k.shape
    assert np.all(np.isfinite(k.astype(np.float32))) and np.all(np.isfinite(v.astype(np.float32)))
    cache = tq.TQCache(B, H, d, T, tq.SideSpec(*ks), tq.SideSpec(vs[0], vs[1], 128))
    cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    out, sc = cache.decode_attention(torch.from_numpy(q).cuda(), T, scores=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode_attention(q, _rows(cache, "k", T), _rows(cache, "v", T))
    ok, worst = rows_close(sc.cpu().numpy(), s_ref)
    print(f"{name} {variant}: scores worst rel {worst:.3e}")
    assert ok, f"scores: worst {worst}"
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    ok, worst = rows_close(got, o_ref)
    print(f"{name} {variant}: out worst rel {worst:.3e}")
    assert ok, f"out: worst {worst}"
