"""GPU tests of the boundary's contract (include/tq.h):

* a decode workspace whose counter region holds garbage decodes correctly
  once tq_decode_workspace_init has run, and every decode leaves the
  counters zero;
* a paged cache whose block table names blocks outside the pools: those
  positions read as zero rows (score 0, value 0) in both decode kernels and
  the dequantizer, appends to them write nothing (both encoders), and every
  other position is as in a contiguous cache whose rows there are zero.
"""
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

S = tq.SideSpec


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tq.lib()


def _env(name, value):
    old = os.environ.get(name)
    os.environ[name] = value
    return old


def _restore(name, old):
    if old is None:
        os.environ.pop(name, None)
    else:
        os.environ[name] = old


@pytest.mark.parametrize("variant", ["auto", "ref"])
def test_workspace_init_clears_garbage_counters(variant):
    old = _env("TQ_DECODE_VARIANT", variant)
    try:
        B, H, Hq, d, T = 2, 4, 16, 128, 3000
        k, v = synth.kv_numpy(5, B, H, T, d, dist="channel", outlier_frac=0.01)
        q = torch.from_numpy(synth.q_numpy(6, B, Hq, d)).cuda()
        cache = tq.TQCache(B, H, d, T, S("packed", 3), S("packed", 4))
        cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
        need = cache.workspace_bytes(Hq, T)
        clean = torch.zeros(need, dtype=torch.uint8, device="cuda")
        ref = cache.decode_attention(q, T, workspace=clean)
        dirty = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        tq.decode_workspace_init(dirty)
        for _ in range(3):
            out = cache.decode_attention(q, T, workspace=dirty)
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
            assert int(dirty[: tq.WORKSPACE_COUNTER_BYTES].view(torch.int32).abs().sum()) == 0
    finally:
        _restore("TQ_DECODE_VARIANT", old)


# 500 positions: an append whose length is not a multiple of 16 (the general
# paged encoder); 512: one that is (the encoder's aligned path, one table
# entry per 16-row tile)
@pytest.mark.parametrize("T", [500, 512], ids=["unaligned", "aligned"])
@pytest.mark.parametrize("qvariant", ["auto", "plain"])
@pytest.mark.parametrize("variant", ["auto", "ref"])
@pytest.mark.parametrize("ks,vs", [(("packed", 3), ("packed", 4)), (("fp16", 0), ("packed", 4)),
                                   (("int8", 0), ("int8", 0))], ids=["tq35", "asym", "int8"])
def test_out_of_range_blocks_read_zero_and_take_no_writes(ks, vs, variant, qvariant, T):
    old_d = _env("TQ_DECODE_VARIANT", variant)
    old_q = _env("TQ_QUANTIZE_VARIANT", qvariant)
    try:
        B, H, Hq, d, bs, cap = 2, 2, 8, 128, 64, 512
        nb = B * cap // bs
        table = torch.from_numpy(np.random.default_rng(2).permutation(nb).astype(np.int32).reshape(B, cap // bs))
        paged = tq.TQCache(B, H, d, cap, S(*ks), S(*vs), block_table=table, block_size=bs, num_blocks=nb)
        # two entries pointing outside the pools, set on the device after the
        # binding's own host check: block 2 of sequence 0 and block 5 of
        # sequence 1 (positions [128, 192) and [320, 384))
        orphans = (int(table[0, 2]), int(table[1, 5]))
        paged.block_table[0, 2] = nb + 5
        paged.block_table[1, 5] = -1
        torch.cuda.synchronize()
        k, v = synth.kv_numpy(9, B, H, T, d, dist="channel", outlier_frac=0.01)
        paged.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
        # the reference: a contiguous cache whose rows in those blocks are zero
        kz, vz = k.copy(), v.copy()
        for x in (kz, vz):
            x[0, :, 128:192] = 0
            x[1, :, 320:384] = 0
        contig = tq.TQCache(B, H, d, cap, S(*ks), S(*vs))
        contig.quantize_append(torch.from_numpy(kz).cuda(), torch.from_numpy(vz).cuda(), 0)
        q = torch.from_numpy(synth.q_numpy(10, B, Hq, d)).cuda()
        out_p, sc_p = paged.decode_attention(q, T, scores=True)
        out_c, sc_c = contig.decode_attention(q, T, scores=True)
        torch.cuda.synchronize()
        # nothing was written to the two pool blocks no valid entry names
        for name, t in paged.tensors.items():
            for blk in orphans:
                assert int(t[blk].abs().sum()) == 0, (name, blk)
        assert torch.equal(sc_p[0, :, 128:192], torch.zeros_like(sc_p[0, :, 128:192]))
        assert torch.equal(sc_p[1, :, 320:384], torch.zeros_like(sc_p[1, :, 320:384]))
        assert torch.equal(sc_p, sc_c)
        assert torch.equal(out_p, out_c)
        for side, spec in (("k", ks), ("v", vs)):
            if spec[0] == "fp16":
                continue
            dq = paged.dequantize(side, 100, 300)
            torch.cuda.synchronize()
            assert int(dq[0, :, 28:92].abs().sum()) == 0 and int(dq[1, :, 220:284].abs().sum()) == 0
            assert torch.equal(dq, contig.dequantize(side, 100, 300))
    finally:
        _restore("TQ_DECODE_VARIANT", old_d)
        _restore("TQ_QUANTIZE_VARIANT", old_q)
