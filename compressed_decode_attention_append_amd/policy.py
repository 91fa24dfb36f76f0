"""Host-side cache policy over the C ABI: which layers get a TurboQuant cache,
in which mode, and when an existing full-precision cache is converted.

Host logic only: every conversion runs through ``TQCache.quantize_append``
(``tq_quantize_append`` in libtq), so nothing here computes on the device by
itself.

What it follows:

* "TurboQuant KV Cache Quantization in MLX-VLM", "Quantization Codecs and Bit
  Splitting": a fractional bit budget b splits floor(b) to K and ceil(b) to V.
* "How to Use TurboQuant with the MLX-VLM CLI", "Cache Quantization Hook" (the
  ``maybe_quantize_kv_cache`` walk-through) and its FAQ "Why does TurboQuant
  skip the last layer?": a layer cache that is already TurboQuant stays as it
  is; an empty full-precision cache is replaced by an empty TurboQuant cache;
  a non-empty one shorter than ``quantized_kv_start`` stays full precision; a
  longer one is converted (``from_cache``); the last layer is never quantized.
  ("TurboQuant KV Cache Quantization in MLX-VLM", "Programmatic API
  Integration", passes ``quantized_kv_start`` to the generation loop.)
* mlxcel "TurboQuant KV cache": "Available modes" (the user-facing mode names:
  fp16, int8, turbo4 / turbo4-sym, fp16+turbo4 / turbo4-asym,
  turbo4-delegated, fp16+turbo3 / turbo3-asym / turbo3; symmetric 3-bit is
  not offered), "CLI
  and server flags" (the supported K/V split-flag combinations) and
  "Boundary-V layer protection" (``--turbo-boundary-v N``: the first N and
  last N layers keep their V cache in fp16 while a Turbo mode is active).

Readings where the pages leave a step open:

* "turbo4-delegated" keeps K in fp16 (the delegated split is a V-side one) with
  a 256-position hot window, the window of the delegated configuration here.
* With boundary-V a layer keeps its mode's K side; if that is fp16 too, the
  layer stays wholly full precision.
* ``int8`` is the per-token absmax cache on both sides (no rotation or
  codebook); boundary-V gives its boundary layers an fp16 V.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple, Union

from . import SideSpec, TQCache, TQError
from . import split_bits as _lib_split_bits

DEFAULT_HOT = 256

# user-facing mode name -> (K side, V side); None = the layer stays fp16
_NAMED = {
    "fp16": None,
    "int8": (SideSpec("int8", 0), SideSpec("int8", 0)),
    "turbo4": (SideSpec("packed", 4), SideSpec("packed", 4)),
    "turbo4-sym": (SideSpec("packed", 4), SideSpec("packed", 4)),
    "fp16+turbo4": (SideSpec("fp16", 0), SideSpec("packed", 4)),
    "turbo4-asym": (SideSpec("fp16", 0), SideSpec("packed", 4)),
    "turbo4-delegated": (SideSpec("fp16", 0), SideSpec("delegated", 4, DEFAULT_HOT)),
    "fp16+turbo3": (SideSpec("fp16", 0), SideSpec("packed", 3)),
    "turbo3-asym": (SideSpec("fp16", 0), SideSpec("packed", 3)),
    "turbo3": (SideSpec("fp16", 0), SideSpec("packed", 3)),
}

Sides = Optional[Tuple[SideSpec, SideSpec]]

# supported (K flag, V flag) pairs -> the mode they select; other pairs are
# rejected
_SPLIT = {
    ("fp16", "fp16"): "fp16",
    ("int8", "int8"): "int8",
    ("fp16", "turbo4"): "fp16+turbo4",
    ("fp16", "turbo4-asym"): "fp16+turbo4",
    ("turbo4", "turbo4"): "turbo4",
    ("fp16", "turbo4-delegated"): "turbo4-delegated",
    ("fp16", "turbo3"): "fp16+turbo3",
    ("fp16", "turbo3-asym"): "fp16+turbo3",
}


def split_flags_mode(cache_type_k: str, cache_type_v: str) -> str:
    """The mode a pair of per-side cache-type flags selects."""
    key = (str(cache_type_k).strip().lower(), str(cache_type_v).strip().lower())
    if key not in _SPLIT:
        raise ValueError(f"unsupported K/V cache-type combination {key}")
    return _SPLIT[key]


def split_bits(bits: float) -> Tuple[int, int]:
    """floor(bits) to K, ceil(bits) to V (a whole number gives both sides
    the same width); each side must land in [1, 8].  The split is the
    library's (tq_split_bits); a budget it rejects raises ValueError."""
    b = float(bits)
    if not math.isfinite(b):
        raise ValueError(f"bit budget {bits!r} is not finite")
    try:
        return _lib_split_bits(b)
    except TQError as e:
        raise ValueError(f"bit budget {bits!r} splits outside 1..8 bits per side ({e})") from None


def mode_sides(mode: Union[str, float, int], hot: int = DEFAULT_HOT) -> Sides:
    """(K, V) side specs of a mode name or a numeric bit budget; None for fp16."""
    if isinstance(mode, (int, float)) and not isinstance(mode, bool):
        kb, vb = split_bits(mode)
        return SideSpec("packed", kb), SideSpec("packed", vb)
    name = str(mode).strip().lower()
    if name not in _NAMED:
        raise ValueError(f"unknown cache mode {mode!r}; known: {', '.join(sorted(_NAMED))}")
    sides = _NAMED[name]
    if sides is None:
        return None
    k, v = sides
    if v.mode == "delegated":
        v = SideSpec("delegated", v.bits, int(hot))
    return SideSpec(k.mode, k.bits, k.hot), SideSpec(v.mode, v.bits, v.hot)


def layer_sides(num_layers: int, mode: Union[str, float, int], skip_last: bool = True,
                boundary_v: int = 0, hot: int = DEFAULT_HOT) -> List[Sides]:
    """Per layer: the (K, V) sides its TurboQuant cache uses, or None where the
    layer stays fp16 (the last layer when ``skip_last``; boundary layers whose
    K side is fp16 as well)."""
    if num_layers < 0 or boundary_v < 0:
        raise ValueError("num_layers and boundary_v must be >= 0")
    base = mode_sides(mode, hot)
    out: List[Sides] = []
    for i in range(num_layers):
        if base is None or (skip_last and i == num_layers - 1):
            out.append(None)
            continue
        k, v = base
        if i < boundary_v or i >= num_layers - boundary_v:
            v = SideSpec("fp16", 0)
        out.append(None if (k.mode == "fp16" and v.mode == "fp16") else (k, v))
    return out


@dataclass
class DenseKV:
    """A full-precision layer cache: fp16 k, v [B][Hkv][capacity][d] on the
    device, positions [0, offset) filled."""
    k: object
    v: object
    offset: int = 0

    @property
    def shape(self):
        return tuple(int(x) for x in self.k.shape)


# actions of the conversion plan
KEEP = "keep"          # already a TurboQuant cache
EMPTY = "empty"        # empty dense cache -> empty TurboQuant cache
DENSE = "dense"        # stays full precision
CONVERT = "convert"    # dense cache converted with from_dense


def plan(offsets: Sequence[Optional[int]], sides: Sequence[Sides], quantized_kv_start: int = 0) -> List[str]:
    """The decision for each layer.  ``offsets[i]`` is the filled length of a
    dense cache, or None for a layer that already holds a TurboQuant cache;
    ``sides[i]`` comes from ``layer_sides`` (None: the layer stays dense)."""
    if len(offsets) != len(sides):
        raise ValueError("offsets and sides differ in length")
    out = []
    for off, sd in zip(offsets, sides):
        if off is None:
            out.append(KEEP)
        elif sd is None:
            out.append(DENSE)
        elif off == 0:
            out.append(EMPTY)
        elif off < quantized_kv_start:
            out.append(DENSE)
        else:
            out.append(CONVERT)
    return out


def from_dense(dense: DenseKV, k: SideSpec, v: SideSpec, seed: int = 0, capacity: Optional[int] = None,
               chunk: int = 4096, stream=None) -> TQCache:
    """A TurboQuant cache holding positions [0, dense.offset) of a dense
    cache (the pages' ``from_cache``): quantize-append in chunks of
    ``chunk`` positions.  ``capacity`` defaults to the dense cache's."""
    B, H, cap, d = dense.shape
    cap = cap if capacity is None else int(capacity)
    if dense.offset > cap:
        raise ValueError(f"offset {dense.offset} exceeds the capacity {cap}")
    out = TQCache(B, H, d, cap, k, v, seed=seed, device=dense.k.device)
    for s in range(0, int(dense.offset), int(chunk)):
        n = min(int(chunk), int(dense.offset) - s)
        out.quantize_append(dense.k[:, :, s:s + n].contiguous(), dense.v[:, :, s:s + n].contiguous(), s,
                            stream=stream)
    return out


def maybe_quantize(caches: Sequence[Union[DenseKV, TQCache]], mode: Union[str, float, int],
                   quantized_kv_start: int = 0, skip_last: bool = True, boundary_v: int = 0,
                   seed: int = 0, hot: int = DEFAULT_HOT, stream=None) -> List[Union[DenseKV, TQCache]]:
    """Apply the layer policy to one model's per-layer caches and return the
    new list (the inputs are not modified)."""
    sides = layer_sides(len(caches), mode, skip_last, boundary_v, hot)
    offsets = [None if isinstance(c, TQCache) else int(c.offset) for c in caches]
    actions = plan(offsets, sides, quantized_kv_start)
    out: List[Union[DenseKV, TQCache]] = []
    for c, sd, act in zip(caches, sides, actions):
        if act in (KEEP, DENSE):
            out.append(c)
        elif act == EMPTY:
            B, H, cap, d = c.shape
            out.append(TQCache(B, H, d, cap, sd[0], sd[1], seed=seed, device=c.k.device))
        else:
            out.append(from_dense(c, sd[0], sd[1], seed=seed, stream=stream))
    return out
