"""Seeded random configurations through the whole path, checked against the
oracle.

Each case draws, from its own seeded generator: a shape (batch, KV heads,
query group of 1 to 16 heads, head_dim), the modes of K and V (packed at several widths,
fp16, INT8, a delegated V), contiguous or paged storage (block size and a
shuffled block table), a run of appends in order (lengths from 1 to a few
hundred, some of them multiples of 16, so both encoders and the aligned and
general paged paths are taken), a decode length and a split count.

Checks, as in the fixed-case parity tests:
* packed sides: the codes the GPU wrote equal the oracle's quantization of
  the same fp16 rows, except within 1e-6 of a threshold (one code apart
  there); norms within 1e-6; INT8 sides: codes and scales equal the exact
  definition; fp16 sides: the rows themselves;
* decode (both kernels): scores and outputs against the oracle's attention
  over the rows the GPU wrote, within 2e-3 of each row's largest magnitude
  (for scores, at least 1e-3 of the row's Cauchy-Schwarz bound: a
  one-position row can cancel to near zero);
* sparse-V (both kernels, a threshold per case): within the oracle's bound
  of the exact output;
* the allocation-free entry point: the same output as the workspace call;
* the fused append-then-attend call: one more position appended and
  attended in one call (one launch or its two-call fallback, as the shape
  decides), the row it wrote and the output against the oracle;
* dequantize of the packed and INT8 sides over a range of positions: the
  oracle's dequantization of the same codes, within 1e-5 of each row's
  largest magnitude.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from parity import codes_agree, rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

S = tq.SideSpec
N_CASES = 40


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


def _draw(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128], p=[0.3, 0.7]))
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16], p=[0.1, 0.1, 0.1, 0.2, 0.1, 0.1, 0.16, 0.07, 0.07]))
    k_mode = str(rng.choice(["packed", "fp16", "int8"], p=[0.6, 0.25, 0.15]))
    v_mode = str(rng.choice(["packed", "fp16", "delegated", "int8"], p=[0.55, 0.1, 0.2, 0.15]))
    bits = lambda: int(rng.choice([1, 2, 3, 4, 5, 8], p=[0.05, 0.15, 0.35, 0.35, 0.05, 0.05]))  # noqa: E731
    # every tenth case has INT8 on both sides (the matrix-core INT8 decode at
    # head_dim 128) and every tenth INT8 K beside another V (the plain kernel)
    if seed % 10 == 3:
        k_mode, v_mode = "int8", "int8"
    elif seed % 10 == 7:
        k_mode = "int8"
    k = S(k_mode, bits() if k_mode == "packed" else 0)
    v = S(v_mode, bits() if v_mode in ("packed", "delegated") else 0, int(rng.choice([32, 64, 256])))
    n_app = int(rng.integers(1, 5))
    lens = []
    for _ in range(n_app):
        n = int(rng.integers(1, 400))
        if rng.random() < 0.5:
            n = max(16, n - n % 16)
        lens.append(n)
    total = sum(lens)
    paged = bool(rng.random() < 0.4)
    bs = int(rng.choice([32, 64, 128]))
    cap = total + int(rng.integers(0, 100))
    if paged:
        cap = -(-cap // bs) * bs
    if v_mode == "delegated":
        length = total
    else:
        length = int(rng.integers(1, total + 1))
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    dist = str(rng.choice(["iid", "channel"]))
    return dict(d=d, B=B, H=H, G=G, k=k, v=v, lens=lens, paged=paged, bs=bs, cap=cap, length=length,
                splits=splits, dist=dist)


def _view(cache, name):
    return cache.logical(name) if cache.paged else cache.tensors[name]


def _check_written(cache, side, spec, x, pos):
    """Rows [pos, pos + n) of one side against the oracle (delegated V is
    checked through the decode only: its rows move between ring and cold
    store as later appends arrive)."""
    n, d = x.shape[2], cache.head_dim
    if spec.mode == "fp16":
        got = _view(cache, side + "_fp16")[:, :, pos:pos + n].cpu().numpy()
        assert np.array_equal(got, x), side
    elif spec.mode == "int8":
        c = _view(cache, side + "_codes")[:, :, pos:pos + n].cpu().numpy().view(np.int8)
        s = _view(cache, side + "_norms")[:, :, pos:pos + n].cpu().numpy()
        c_o, s_o = oracle.int8_quantize(x)
        assert np.array_equal(c, c_o) and np.array_equal(s, s_o), side
    elif spec.mode == "packed":
        R = oracle.rotation_matrix(cache.seed, d)
        _, t = oracle.lloyd_max(d, spec.bits)
        codes_o, n_o, y_o = oracle.quantize(x, R, t)
        words = _view(cache, side + "_codes")[:, :, pos:pos + n].cpu().numpy()
        norms = _view(cache, side + "_norms")[:, :, pos:pos + n].cpu().numpy()
        got = words_to_codes(words, spec.bits, d)
        ok, ndiff, nnear = codes_agree(got, codes_o, y_o, t)
        assert ok, f"{side}: {ndiff} codes differ outside the threshold band ({nnear} near)"
        assert np.all(np.abs(norms - n_o) <= 1e-6 * np.maximum(n_o, 1e-30)), side


def _rows(cache, side, spec, length):
    """float64 rows [0, length) of one side as the decode must see them."""
    d = cache.head_dim
    if spec.mode == "fp16":
        return _view(cache, side + "_fp16")[:, :, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        c = _view(cache, side + "_codes")[:, :, :length].cpu().numpy().view(np.int8)
        return oracle.int8_dequantize(c, _view(cache, side + "_norms")[:, :, :length].cpu().numpy())
    R = oracle.rotation_matrix(cache.seed, d)
    cb, _ = oracle.lloyd_max(d, spec.bits)

    def packed(lo, hi):
        words = _view(cache, side + "_codes")[:, :, lo:hi].cpu().numpy()
        norms = _view(cache, side + "_norms")[:, :, lo:hi].cpu().numpy().astype(np.float64)
        return oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, cb)

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


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    c = _draw(5000 + seed)
    d, B, H, G = c["d"], c["B"], c["H"], c["G"]
    Hq = H * G
    desc = (f"seed {seed}: B{B} Hkv{H} G{G} d{d} K {c['k'].mode}{c['k'].bits} "
            f"V {c['v'].mode}{c['v'].bits}{'/hot ' + str(c['v'].hot) if c['v'].mode == 'delegated' else ''} "
            f"appends {c['lens']} cap {c['cap']} {'paged bs ' + str(c['bs']) if c['paged'] else 'contiguous'} "
            f"length {c['length']} splits {c['splits']} {c['dist']}")
    print(desc, flush=True)
    kw = {}
    if c["paged"]:
        mb = c["cap"] // c["bs"]
        nb = B * mb + 2
        table = np.random.default_rng(seed).permutation(nb)[:B * mb].reshape(B, mb).astype(np.int32)
        kw = dict(block_table=torch.from_numpy(table), block_size=c["bs"], num_blocks=nb)
    cache = tq.TQCache(B, H, d, c["cap"], c["k"], c["v"], device="cuda", **kw)
    pos = 0
    for i, n in enumerate(c["lens"]):
        k, v = synth.kv_numpy(7000 + 10 * seed + i, B, H, n, d, dist=c["dist"], outlier_frac=0.01)
        cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), pos)
        torch.cuda.synchronize()
        _check_written(cache, "k", c["k"], k, pos)
        if c["v"].mode != "delegated":
            _check_written(cache, "v", c["v"], v, pos)
        pos += n
    T = c["length"]
    q = synth.q_numpy(9000 + seed, B, Hq, d)
    kr, vr = _rows(cache, "k", c["k"], T), _rows(cache, "v", c["v"], T)
    o_ref, s_ref = oracle.decode_attention(q, kr, vr)
    # scores: a row's scale is at least 1e-3 of the Cauchy-Schwarz bound
    # |q_h| max_i |k_i| / sqrt(d) of its dot products (the scale of the terms
    # each sums), so a short row that cancels to near zero is not judged by
    # its own magnitude alone
    kmax = np.max(np.linalg.norm(kr, axis=-1), axis=-1) if T else np.zeros((B, H))
    s_floor = 1e-3 * np.linalg.norm(q.astype(np.float64), axis=-1) * np.repeat(kmax, G, axis=1) / np.sqrt(d)
    tau = (1e-4, 1e-3, 1e-2)[seed % 3]
    bound = oracle.sparse_v_bound(q, kr, vr, tau)
    qd = torch.from_numpy(q).cuda()
    old = os.environ.get("TQ_DECODE_VARIANT")
    try:
        for variant in ("auto", "ref"):
            os.environ["TQ_DECODE_VARIANT"] = variant
            out, sc = cache.decode_attention(qd, T, n_splits=c["splits"], scores=True)
            sparse = cache.decode_attention(qd, T, n_splits=c["splits"], sparse_v=tau)
            torch.cuda.synchronize()
            ok_s, worst_s = rows_close(sc.cpu().numpy(), s_ref, floor=s_floor)
            ok_o, worst_o = rows_close(out.cpu().numpy(), o_ref)
            print(f"  {variant}: scores {worst_s:.2e}, out {worst_o:.2e}", flush=True)
            assert ok_s, f"{desc} [{variant}]: scores worst {worst_s}"
            assert ok_o, f"{desc} [{variant}]: out worst {worst_o}"
            exact = out.cpu().numpy().astype(np.float64)
            scale = np.max(np.abs(exact), axis=-1, keepdims=True)
            moved = np.abs(sparse.cpu().numpy().astype(np.float64) - exact)
            assert np.all(moved <= bound * (1 + 1e-3) + 1e-5 * scale), f"{desc} [{variant}]: sparse-V tau {tau}"
            if variant == "auto":
                free = cache.decode_attention_noalloc(qd, T, n_splits=c["splits"])
                torch.cuda.synchronize()
                assert torch.equal(free, out), f"{desc}: allocation-free call differs"
        # one more position through the fused call, attended at once
        pos = sum(c["lens"])
        if pos < c["cap"] and (c["v"].mode != "delegated" or T == pos):
            kn, vn = synth.kv_numpy(8000 + seed, B, H, 1, d, dist=c["dist"], outlier_frac=0.01)
            os.environ["TQ_DECODE_VARIANT"] = "auto"
            out_f = cache.decode_attention_append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), pos, qd,
                                                  pos + 1, n_splits=c["splits"])
            torch.cuda.synchronize()
            _check_written(cache, "k", c["k"], kn, pos)
            if c["v"].mode != "delegated":
                _check_written(cache, "v", c["v"], vn, pos)
            o_f, _ = oracle.decode_attention(q, _rows(cache, "k", c["k"], pos + 1), _rows(cache, "v", c["v"], pos + 1))
            ok_f, worst_f = rows_close(out_f.cpu().numpy(), o_f)
            print(f"  fused append at {pos}: out {worst_f:.2e}", flush=True)
            assert ok_f, f"{desc}: fused append-then-attend worst {worst_f}"
        rng = np.random.default_rng(seed + 77)
        for side, spec, rows in (("k", c["k"], kr), ("v", c["v"], vr)):
            if spec.mode in ("packed", "int8"):
                st = int(rng.integers(0, T))
                cnt = int(rng.integers(1, T - st + 1))
                dq = cache.dequantize(side, st, cnt)
                torch.cuda.synchronize()
                ok, worst = rows_close(dq.cpu().numpy(), rows[:, :, st:st + cnt], 1e-5)
                assert ok, f"{desc}: dequantize {side} [{st}, {st + cnt}) worst {worst}"
    finally:
        if old is None:
            os.environ.pop("TQ_DECODE_VARIANT", None)
        else:
            os.environ["TQ_DECODE_VARIANT"] = old
