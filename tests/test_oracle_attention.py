"""Pins for the oracle's attention and cache bookkeeping.

Checked against: torch's scaled_dot_product_attention (CPU, float64, K/V
repeated per query group), the special cases T = 1 and identical keys, the
rotated-domain identities that license scoring and accumulating on codes, and
direct quantization of the evicted tokens for the delegated ring.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _sdpa(q, k, v):
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    qt = torch.from_numpy(q)[:, :, None, :]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0, :].numpy()


@pytest.mark.parametrize("B,Hkv,Hq,T,d", [(1, 2, 4, 256, 64), (2, 4, 32, 77, 128), (1, 1, 1, 1, 32)])
def test_attention_matches_torch_sdpa(B, Hkv, Hq, T, d):
    rng = np.random.default_rng(T + d)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    out, s = oracle.attention(q, k, v)
    assert np.allclose(out, _sdpa(q, k, v), rtol=1e-12, atol=1e-12)
    G = Hq // Hkv
    assert np.allclose(s[0, 0], k[0, 0] @ q[0, 0] / math.sqrt(d))
    assert np.allclose(s[0, G - 1], k[0, 0] @ q[0, G - 1] / math.sqrt(d))


def test_attention_special_cases():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 16))
    v = rng.standard_normal((1, 1, 5, 16))
    k1 = rng.standard_normal((1, 1, 1, 16))
    out, _ = oracle.attention(q, k1, v[:, :, :1])
    assert np.allclose(out[0, 0], v[0, 0, 0]) and np.allclose(out[0, 1], v[0, 0, 0])
    k = np.repeat(k1, 5, axis=2)
    out, _ = oracle.attention(q, k, v)
    assert np.allclose(out[0, 1], v[0, 0].mean(axis=0))


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4)])
def test_rotated_domain_identities(d, bits):
    """n <R q, c[code]> / sqrt(d) equals q . dequant / sqrt(d), and
    R^T (sum_i p_i n_i c[code_i]) equals sum_i p_i dequant_i."""
    k, v = synth.kv_numpy(11, 1, 1, 64, d, dist="channel", outlier_frac=0.02)
    q = synth.q_numpy(11, 1, 1, d).astype(np.float64)[0, 0]
    R = oracle.rotation_matrix(0, d)
    c, t = oracle.lloyd_max(d, bits)
    codes, n, _ = oracle.quantize(k[0, 0], R, t)
    kt = oracle.dequantize(codes, n, R, c)
    plain = kt @ q / math.sqrt(d)
    fused = n * (c[codes] @ (R @ q)) / math.sqrt(d)
    assert np.max(np.abs(fused - plain)) <= 1e-12 * np.max(np.abs(plain))
    p = np.exp(plain - plain.max()); p /= p.sum()
    vcodes, vn, _ = oracle.quantize(v[0, 0], R, t)
    vt = oracle.dequantize(vcodes, vn, R, c)
    acc_rot = (p * vn) @ c[vcodes]
    assert np.max(np.abs(acc_rot @ R - p @ vt)) <= 1e-12 * np.max(np.abs(p @ vt))


@pytest.mark.parametrize("chunks", [[300], [1] * 40 + [260], [100, 100, 100], [255, 1, 2, 42]])
def test_delegated_ring_bookkeeping(chunks):
    hot, d = 64, 32
    T = sum(chunks)
    k, v = synth.kv_numpy(2, 2, 3, T, d)
    side = oracle.DelegatedSide(2, 3, T, d, 4, seed=0, hot=hot)
    off = 0
    for n in chunks:
        side.append(v[:, :, off:off + n], off)
        off += n
    n_cold = T - hot
    codes, norms, _ = oracle.quantize(v[:, :, :n_cold], side.cold.R, side.cold.thresholds)
    assert np.array_equal(side.cold.codes[:, :, :n_cold], codes)
    assert np.array_equal(side.cold.norms[:, :, :n_cold], norms.astype(np.float32))
    assert np.all(side.cold.codes[:, :, n_cold:] == 0)
    for p in range(n_cold, T):
        assert np.array_equal(side.ring[:, :, p % hot], v[:, :, p])
    rows = side.rows(T)
    assert np.array_equal(rows[:, :, n_cold:], v[:, :, n_cold:].astype(np.float64))


def test_delegated_short_context_is_plain_fp16_attention():
    hot, d = 256, 64
    k, v = synth.kv_numpy(4, 1, 2, 200, d)
    q = synth.q_numpy(4, 1, 4, d)
    side = oracle.DelegatedSide(1, 2, 200, d, 4, seed=0, hot=hot)
    side.append(v, 0)
    out, _ = oracle.decode_attention(q, k.astype(np.float64), side.rows(200))
    assert np.allclose(out, _sdpa(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)), atol=1e-12)


def test_packed_side_writes_only_its_rows():
    k, _ = synth.kv_numpy(5, 1, 2, 40, 64)
    side = oracle.PackedSide(1, 2, 100, 64, 3, seed=0)
    side.write(k[:, :, :10], 0)
    side.write(k[:, :, 10:40], 10)
    assert np.all(side.codes[:, :, 40:] == 0) and np.all(side.norms[:, :, 40:] == 0)
    codes, n, _ = oracle.quantize(k, side.R, side.thresholds)
    assert np.array_equal(side.codes[:, :, :40], codes)


# ---- sparse-V bound (mlxcel "TurboQuant KV cache", sparse-V threshold) ----

def test_sparse_v_bound_hand_case():
    # two positions, scores 0 and -10 ln 2 (relative weights 1 and 2^-10):
    # with tau = 1e-2 the second is dropped; by hand the bound is
    # 2^-10 |v_1| / (1 + 2^-10) and the sparse output p_0 v_0 / (1 + 2^-10)
    d = 4
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 2, d))
    k[0, 0, 1, 0] = -10.0 * np.log(2.0) * np.sqrt(d)
    v = np.array([[[[1.0, -2.0, 3.0, 0.5], [-4.0, 8.0, 0.25, -1.0]]]])
    w = 2.0 ** -10
    b = oracle.sparse_v_bound(q, k, v, 1e-2)
    assert np.allclose(b[0, 0], w * np.abs(v[0, 0, 1]) / (1 + w), rtol=1e-14, atol=0)
    o = oracle.sparse_v_attention(q, k, v, 1e-2)
    assert np.allclose(o[0, 0], v[0, 0, 0] / (1 + w), rtol=1e-14, atol=0)
    # a threshold below both weights drops nothing
    assert np.all(oracle.sparse_v_bound(q, k, v, w / 2) == 0)


def test_sparse_v_zero_threshold_is_exact():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 16))
    k = rng.standard_normal((2, 2, 50, 16))
    v = rng.standard_normal((2, 2, 50, 16))
    assert np.all(oracle.sparse_v_bound(q, k, v, 0.0) == 0)
    o, _ = oracle.attention(q, k, v)
    assert np.allclose(oracle.sparse_v_attention(q, k, v, 0.0), o, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("tau", [1e-3, 0.05, 0.5, 0.99])
def test_sparse_v_drop_stays_within_bound(tau):
    # the largest allowed drop, and a random subset of it, both move every
    # output element by no more than the bound
    rng = np.random.default_rng(int(tau * 1e4))
    q = 3.0 * rng.standard_normal((1, 4, 32))
    k = rng.standard_normal((1, 2, 200, 32))
    v = rng.standard_normal((1, 2, 200, 32))
    o, _ = oracle.attention(q, k, v)
    b = oracle.sparse_v_bound(q, k, v, tau)
    full = oracle.sparse_v_attention(q, k, v, tau)
    assert np.all(np.abs(full - o) <= b * (1 + 1e-12) + 1e-15)
    # a random subset of the droppable positions (rebuilt from the definition)
    G = 2
    for h in range(4):
        s = k[0, h // G] @ q[0, h] / np.sqrt(32)
        p = np.exp(s - s.max())
        drop = (p < tau) & (rng.random(200) < 0.5)
        part = (p[~drop] @ v[0, h // G][~drop]) / p.sum()
        assert np.all(np.abs(part - o[0, h]) <= b[0, h] * (1 + 1e-12) + 1e-15)
