"""The allocation-free decode (tq_decode_attention_noalloc: the library's
fixed per-GPU scratch instead of a caller's workspace) against
tq_decode_attention with a workspace, through the C ABI: two calls in a row,
the second on a smaller input, each bit-identical in outputs and scaled
logits (the same kernels and splits), through both decode kernels.  Run last
(the scratch keeps the counters of whichever call ran before)."""
import os

import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import compressed_decode_attention_append_amd as tq  # noqa: E402

S = tq.SideSpec

# batch, KV heads, query heads, head_dim, positions, K side, V side
CALLS = [
    (2, 8, 32, 128, 9000, ("packed", 3), ("packed", 4)),
    (1, 2, 8, 128, 700, ("fp16", 0), ("packed", 4)),
]


@pytest.mark.parametrize("variant", ["auto", "ref"])
def test_noalloc_matches_workspace_decode(variant):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    old = os.environ.get("TQ_DECODE_VARIANT")
    os.environ["TQ_DECODE_VARIANT"] = variant
    try:
        for i, (B, H, Hq, d, T, ks, vs) in enumerate(CALLS):
            print(f"noalloc call {i}: B{B} H{H} Hq{Hq} d{d} T{T} {ks} {vs} ({variant})", flush=True)
            k, v = synth.kv_numpy(40 + i, B, H, T, d, dist="channel", outlier_frac=0.01)
            q = torch.from_numpy(synth.q_numpy(50 + i, B, Hq, d)).cuda()
            cache = tq.TQCache(B, H, d, T, S(*ks), S(*vs))
            cache.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
            assert cache.workspace_bytes(Hq, T) <= tq.TQ_NOALLOC_SCRATCH_BYTES
            ref, sref = cache.decode_attention(q, T, scores=True)
            got, sgot = cache.decode_attention_noalloc(q, T, scores=True)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), f"call {i}: outputs differ"
            assert torch.equal(sgot, sref), f"call {i}: scores differ"
            # an explicit split count through the scratch as well
            got3 = cache.decode_attention_noalloc(q, T, n_splits=3)
            ref3 = cache.decode_attention(q, T, n_splits=3)
            torch.cuda.synchronize()
            assert torch.equal(got3, ref3), f"call {i}: three splits differ"
    finally:
        if old is None:
            os.environ.pop("TQ_DECODE_VARIANT", None)
        else:
            os.environ["TQ_DECODE_VARIANT"] = old
