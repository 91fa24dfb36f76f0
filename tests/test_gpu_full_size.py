"""Parity at the full workload sizes, in the launch configuration the bench
times (library-chosen splits, one layer of each workload).

The whole cache is quantized and attended on the GPU.  The oracle checks
sampled parts it can compute in seconds:

* the codes and norms of a slice of rows of sampled (batch, KV head) units,
  against the oracle's quantization of the same fp16 rows;
* every query head of sampled units: the decode output and the scaled
  logits against float64 attention over the rows the oracle rebuilds from
  what the GPU wrote (dequantized packed rows, INT8 rows, fp16 rows as
  stored, the delegated ring).  The outputs come from the call the bench
  times (no score output); a second call with the score output must give
  bit-identical outputs.

Two configurations state their K/V distribution as "the same as config 1",
which reads either as the i.i.d. N(0, 1) rows of the first configuration or
as the log-normal channel scales of the second; both readings run here at the
asymmetric 16K and the 3.5-bit 32K shapes.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import codes_agree, rows_close, words_to_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

# name: batch, KV heads, query heads, head_dim, context, K side, V side, hot,
# distribution, outlier fraction, positions appended in the timed step
FULL = {
    "c2_sym4_4k": (1, 8, 32, 128, 4096, ("packed", 4), ("packed", 4), 0, "channel", 0.01, 0),
    "c3_asym_16k": (8, 8, 32, 128, 16384, ("fp16", 0), ("packed", 4), 0, "channel", 0.01, 1),
    "c3_asym_16k_iid": (8, 8, 32, 128, 16384, ("fp16", 0), ("packed", 4), 0, "iid", 0.0, 1),
    "c4_tq35_32k": (4, 8, 32, 128, 32768, ("packed", 3), ("packed", 4), 0, "channel", 0.01, 8192),
    "c4_tq35_32k_iid": (4, 8, 32, 128, 32768, ("packed", 3), ("packed", 4), 0, "iid", 0.0, 8192),
    "c5_delegated_64k": (16, 4, 32, 128, 65536, ("fp16", 0), ("delegated", 4), 256, "channel", 0.0, 0),
    # the pages' int8 mode at the asymmetric shape (a comparison workload)
    "c3_int8_16k": (8, 8, 32, 128, 16384, ("int8", 0), ("int8", 0), 0, "channel", 0.01, 1),
    # the pages' turbo3-asym mode (fp16 K, 3-bit V) at the same shape
    "c3_turbo3_asym_16k": (8, 8, 32, 128, 16384, ("fp16", 0), ("packed", 3), 0, "channel", 0.01, 1),
    # 2.5 bits (2-bit K, 3-bit V) at the 32K shape
    "c4_tq25_32k": (4, 8, 32, 128, 32768, ("packed", 2), ("packed", 3), 0, "channel", 0.01, 8192),
    # 16 query heads per KV head (head groups) at the 32K shape
    "c4_tq35_32k_g16": (4, 4, 64, 128, 32768, ("packed", 3), ("packed", 4), 0, "channel", 0.01, 8192),
}


def _unit_rows(cache, side, b, h, length):
    """float64 rows [0, length) of one (batch, KV head) unit of one side, as
    the decode must see them, rebuilt from what the GPU wrote."""
    spec = cache.k_spec if side == "k" else cache.v_spec
    d = cache.head_dim
    if spec.mode == "fp16":
        return cache.tensors[side + "_fp16"][b, h, :length].cpu().numpy().astype(np.float64)
    if spec.mode == "int8":
        codes = cache.tensors[side + "_codes"][b, h, :length].cpu().numpy().view(np.int8)
        return oracle.int8_dequantize(codes, cache.tensors[side + "_norms"][b, h, :length].cpu().numpy())
    R = oracle.rotation_matrix(cache.seed, d)
    c, _ = oracle.lloyd_max(d, spec.bits)
    n_cold = length if spec.mode == "packed" else max(0, length - spec.hot)
    out = np.zeros((length, d))
    if n_cold:
        words = cache.tensors[side + "_codes"][b, h, :n_cold].cpu().numpy()
        norms = cache.tensors[side + "_norms"][b, h, :n_cold].cpu().numpy().astype(np.float64)
        out[:n_cold] = oracle.dequantize(words_to_codes(words, spec.bits, d), norms, R, c)
    if spec.mode == "delegated":
        ring = cache.tensors[side + "_ring"][b, h].cpu().numpy()
        for p in range(n_cold, length):
            out[p] = ring[p % spec.hot].astype(np.float64)
    return out


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    B, Hkv, Hq, d, T, ks, vs, hot, dist, outl, n_new = FULL[name]
    G = Hq // Hkv
    kspec = tq.SideSpec(ks[0], ks[1])
    vspec = tq.SideSpec(vs[0], vs[1], hot or 256)
    cache = tq.TQCache(B, Hkv, d, T, kspec, vspec, seed=0, device="cuda:0")
    base = T - n_new
    chunk = 4096
    samples = {}  # (b, h) -> (start, fp16 K rows, fp16 V rows) kept for the code checks
    pick = [(0, 0), (B - 1, Hkv - 1)]
    for s in range(0, base, chunk):
        n = min(chunk, base - s)
        k, v = synth.kv_torch(1009 + s, B, Hkv, n, d, dist=dist, outlier_frac=outl, device="cuda:0")
        cache.quantize_append(k, v, s)
        if s == 0:
            for (b, h) in pick:
                samples[(b, h)] = (0, k[b, h, :512].cpu().numpy(), v[b, h, :512].cpu().numpy())
        del k, v
    if n_new:
        k, v = synth.kv_torch(4243, B, Hkv, n_new, d, dist=dist, outlier_frac=outl, device="cuda:0")
        cache.quantize_append(k, v, base)  # the timed append: one prefill chunk or one token
        if n_new >= 512:
            for (b, h) in pick:
                samples[(b, h, "new")] = (base, k[b, h, :512].cpu().numpy(), v[b, h, :512].cpu().numpy())
        del k, v
    q = synth.q_torch(77, B, Hq, d, device="cuda:0")
    out = cache.decode_attention(q, T)                   # as the bench calls it
    out2, sc = cache.decode_attention(q, T, scores=True)  # the same, with the logits
    torch.cuda.synchronize()
    assert torch.equal(out, out2)

    # codes and norms of sampled rows
    for key, (start, krows, vrows) in samples.items():
        b, h = key[0], key[1]
        for side, spec, rows in (("k", kspec, krows), ("v", vspec, vrows)):
            if spec.mode == "int8":
                c_o, s_o = oracle.int8_quantize(rows)
                got = cache.tensors[side + "_codes"][b, h, start:start + rows.shape[0]].cpu().numpy().view(np.int8)
                sc_got = cache.tensors[side + "_norms"][b, h, start:start + rows.shape[0]].cpu().numpy()
                assert np.array_equal(got, c_o), f"{name} {side} ({b},{h}): {int(np.sum(got != c_o))} codes differ"
                assert np.array_equal(sc_got, s_o)
                continue
            if spec.mode != "packed":
                continue
            R = oracle.rotation_matrix(0, d)
            _, t = oracle.lloyd_max(d, spec.bits)
            codes_o, n_o, y_o = oracle.quantize(rows[None, None], R, t)
            words = cache.tensors[side + "_codes"][b, h, start:start + rows.shape[0]].cpu().numpy()
            got = words_to_codes(words[None, None], spec.bits, d)
            ok, ndiff, nnear = codes_agree(got, codes_o, y_o, t)
            assert ok, f"{name} {side} ({b},{h}) rows {start}+: {ndiff} codes off ({nnear} near a threshold)"
            norms = cache.tensors[side + "_norms"][b, h, start:start + rows.shape[0]].cpu().numpy()
            assert np.all(np.abs(norms - n_o[0, 0]) <= 1e-6 * n_o[0, 0] + 1e-30)

    # decode outputs and logits of every query head of the sampled units
    qn = q.cpu().numpy()
    got = out.cpu().numpy()
    for (b, h) in pick:
        kr = _unit_rows(cache, "k", b, h, T)[None, None]
        vr = _unit_rows(cache, "v", b, h, T)[None, None]
        heads = slice(h * G, (h + 1) * G)
        o_ref, s_ref = oracle.decode_attention(qn[b:b + 1, heads], kr, vr)
        ok, worst = rows_close(sc[b, heads].cpu().numpy(), s_ref[0])
        print(f"{name} unit ({b},{h}): scores worst rel {worst:.3e}")
        assert ok, f"{name} unit ({b},{h}): scores worst {worst}"
        ok, worst = rows_close(got[b, heads], o_ref[0])
        print(f"{name} unit ({b},{h}): out worst rel {worst:.3e}")
        assert ok, f"{name} unit ({b},{h}): worst {worst}"


@pytest.mark.parametrize("name", ["c4_tq35_32k", "c3_asym_16k", "c5_delegated_64k"])
def test_full_size_paged_matches_contiguous(name):
    # the same appends into a contiguous cache and a paged one (blocks of 256
    # positions in a random order): decode outputs bit-identical, and the
    # storage equal at every logical position of sampled units
    B, Hkv, Hq, d, T, ks, vs, hot, dist, outl, n_new = FULL[name]
    kspec = tq.SideSpec(ks[0], ks[1])
    vspec = tq.SideSpec(vs[0], vs[1], hot or 256)
    bs = 256
    nb = B * (T // bs)
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(3)).to(torch.int32).reshape(B, T // bs)
    contig = tq.TQCache(B, Hkv, d, T, kspec, vspec, seed=0, device="cuda:0")
    paged = tq.TQCache(B, Hkv, d, T, kspec, vspec, seed=0, device="cuda:0", block_table=perm, block_size=bs,
                       num_blocks=nb)
    base = T - n_new
    for s in range(0, base, 4096):
        n = min(4096, base - s)
        k, v = synth.kv_torch(2003 + s, B, Hkv, n, d, dist=dist, outlier_frac=outl, device="cuda:0")
        contig.quantize_append(k, v, s)
        paged.quantize_append(k, v, s)
        del k, v
    if n_new:
        k, v = synth.kv_torch(4243, B, Hkv, n_new, d, dist=dist, outlier_frac=outl, device="cuda:0")
        contig.quantize_append(k, v, base)
        paged.quantize_append(k, v, base)
        del k, v
    q = synth.q_torch(78, B, Hq, d, device="cuda:0")
    oc = contig.decode_attention(q, T)
    op = paged.decode_attention(q, T)
    torch.cuda.synchronize()
    assert torch.equal(oc, op)
    for name_t in contig.tensors:
        lv = paged.logical(name_t)
        for (b, h) in ((0, 0), (B - 1, Hkv - 1)):
            assert torch.equal(contig.tensors[name_t][b, h], lv[b, h]), (name_t, b, h)
