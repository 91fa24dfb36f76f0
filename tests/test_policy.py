"""Host-side cache policy (no device work): mode names, bit splits, layer
plans and conversion decisions, checked against what the pages state."""
import pytest

from compressed_decode_attention_append_amd import SideSpec
from compressed_decode_attention_append_amd import policy as P


def _sides(k_mode, k_bits, v_mode, v_bits):
    return (k_mode, k_bits, v_mode, v_bits)


def _flat(s):
    if s is None:
        return None
    k, v = s
    return _sides(k.mode, k.bits if k.mode != "fp16" else 0, v.mode, v.bits if v.mode != "fp16" else 0)


# "Quantization Codecs and Bit Splitting": floor to K, ceil to V; the pages'
# own example budget is 3.5 bits, and other fractions are split literally
# (4.2 -> K4 / V5).  The policy's split is the library's tq_split_bits.
@pytest.mark.parametrize("bits,k,v", [(3.5, 3, 4), (3, 3, 3), (4, 4, 4), (4.2, 4, 5), (1.5, 1, 2), (7.5, 7, 8),
                                      (2.0, 2, 2)])
def test_split_bits(bits, k, v):
    assert P.split_bits(bits) == (k, v) == P._lib_split_bits(bits)
    assert _flat(P.mode_sides(bits)) == _sides("packed", k, "packed", v)


@pytest.mark.parametrize("bits", [0.5, 8.5, 9, float("nan"), float("inf")])
def test_split_bits_out_of_range(bits):
    with pytest.raises(ValueError):
        P.split_bits(bits)


# mlxcel "Available modes"
@pytest.mark.parametrize("name,want", [
    ("fp16", None),
    ("int8", _sides("int8", 0, "int8", 0)),
    ("turbo4", _sides("packed", 4, "packed", 4)),
    ("turbo4-sym", _sides("packed", 4, "packed", 4)),
    ("fp16+turbo4", _sides("fp16", 0, "packed", 4)),
    ("turbo4-asym", _sides("fp16", 0, "packed", 4)),
    ("turbo4-delegated", _sides("fp16", 0, "delegated", 4)),
    ("fp16+turbo3", _sides("fp16", 0, "packed", 3)),
    ("turbo3-asym", _sides("fp16", 0, "packed", 3)),
    ("turbo3", _sides("fp16", 0, "packed", 3)),   # symmetric 3-bit is not offered
    ("  Turbo4-ASYM ", _sides("fp16", 0, "packed", 4)),
])
def test_named_modes(name, want):
    assert _flat(P.mode_sides(name)) == want


def test_delegated_hot_window():
    k, v = P.mode_sides("turbo4-delegated", hot=64)
    assert (v.mode, v.bits, v.hot) == ("delegated", 4, 64)
    assert P.mode_sides("turbo4-delegated")[1].hot == 256


@pytest.mark.parametrize("name", ["turbo5", "turbo3-sym", "int4", ""])
def test_rejected_modes(name):
    with pytest.raises(ValueError):
        P.mode_sides(name)


# "CLI and server flags": the supported split-flag combinations
@pytest.mark.parametrize("k,v,mode", [("fp16", "fp16", "fp16"), ("int8", "int8", "int8"),
                                      ("fp16", "turbo4", "fp16+turbo4"), ("fp16", "turbo4-asym", "fp16+turbo4"),
                                      ("turbo4", "turbo4", "turbo4"), ("fp16", "turbo4-delegated", "turbo4-delegated"),
                                      ("fp16", "turbo3", "fp16+turbo3"), ("fp16", "turbo3-asym", "fp16+turbo3")])
def test_split_flags(k, v, mode):
    assert P.split_flags_mode(k, v) == mode


@pytest.mark.parametrize("k,v", [("turbo4", "fp16"), ("turbo3", "turbo3"), ("int8", "fp16"), ("fp16", "int8")])
def test_split_flags_unsupported(k, v):
    with pytest.raises(ValueError):
        P.split_flags_mode(k, v)


def test_last_layer_skipped():
    # "Why does TurboQuant skip the last layer?"
    plan = P.layer_sides(5, 3.5)
    assert [p is None for p in plan] == [False, False, False, False, True]
    assert all(_flat(p) == _sides("packed", 3, "packed", 4) for p in plan[:4])
    assert P.layer_sides(5, 3.5, skip_last=False)[4] is not None
    assert P.layer_sides(1, "turbo4") == [None]
    assert P.layer_sides(0, "turbo4") == []


def test_boundary_v():
    # "Boundary-V layer protection": first N and last N layers keep V in fp16
    plan = P.layer_sides(8, "turbo4", skip_last=False, boundary_v=2)
    kinds = [_flat(p) for p in plan]
    fp16v = _sides("packed", 4, "fp16", 0)
    both = _sides("packed", 4, "packed", 4)
    assert kinds == [fp16v, fp16v, both, both, both, both, fp16v, fp16v]
    # with an fp16 K the boundary layers stay wholly full precision
    plan = P.layer_sides(6, "fp16+turbo4", skip_last=True, boundary_v=1)
    assert [p is None for p in plan] == [True, False, False, False, False, True]
    # a boundary wider than half the model covers every layer
    assert all(_flat(p) == fp16v for p in P.layer_sides(3, "turbo4", skip_last=False, boundary_v=5))
    with pytest.raises(ValueError):
        P.layer_sides(3, "turbo4", boundary_v=-1)


def test_fp16_mode_keeps_everything_dense():
    assert P.layer_sides(4, "fp16", skip_last=False) == [None] * 4
    assert P.plan([0, 10, None], [None, None, None]) == [P.DENSE, P.DENSE, P.KEEP]


def test_plan_follows_the_hook():
    # "Cache Quantization Hook": TurboQuant entries stay; empty dense -> new
    # TurboQuant cache; shorter than quantized_kv_start -> stays dense; else
    # converted.  The boundary at exactly quantized_kv_start converts.
    sd = (SideSpec("packed", 3), SideSpec("packed", 4))
    offsets = [None, 0, 1, 4999, 5000, 9000, 0]
    sides = [sd] * 6 + [None]
    assert P.plan(offsets, sides, quantized_kv_start=5000) == [
        P.KEEP, P.EMPTY, P.DENSE, P.DENSE, P.CONVERT, P.CONVERT, P.DENSE]
    # quantized_kv_start = 0: every non-empty dense cache converts
    assert P.plan([3, 0], [sd, sd]) == [P.CONVERT, P.EMPTY]
    with pytest.raises(ValueError):
        P.plan([0], [sd, sd])
