"""Seeded synthetic K/V/q inputs for the TurboQuant cache workloads.

This module only draws random numbers. It holds none of the method's
arithmetic (no norm, rotation, codebook, packing or attention), so the CPU
oracle and the HIP path can both be fed from it without sharing code.

Two distributions are provided, following the workload descriptions:

* ``iid``: every element of K, V and q is N(0, 1), rounded to fp16.
* ``channel``: K and V elements are ``scale[h, j] * N(0, 1)`` with a
  per-(head, channel) scale ``exp(0.5 * z)``, ``z ~ N(0, 1)`` (a log-normal
  with sigma 0.5), fixed across batch and tokens and drawn separately for K
  and V.  Optionally ``round(outlier_frac * H * d)`` distinct (head, channel)
  pairs, drawn without replacement, get their scale multiplied by
  ``outlier_scale``.  Elements are formed in fp32 and rounded to fp16
  (round-to-nearest-even).  q stays N(0, 1).

Layouts: K and V are ``[B, H, T, d]``; q is ``[B, Hq, d]``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "channel_scales",
    "kv_numpy",
    "q_numpy",
    "kv_torch",
    "q_torch",
    "CONFIGS",
]


def channel_scales(rng: np.random.Generator, heads: int, head_dim: int,
                   outlier_frac: float, outlier_scale: float,
                   sigma: float = 0.5) -> np.ndarray:
    """Per-(head, channel) scales, shape [heads, head_dim], float32."""
    z = rng.standard_normal((heads, head_dim))
    s = np.exp(sigma * z)
    n_out = int(round(outlier_frac * heads * head_dim))
    if n_out > 0:
        flat = rng.choice(heads * head_dim, size=n_out, replace=False)
        s.reshape(-1)[flat] *= outlier_scale
    return s.astype(np.float32)


def kv_numpy(seed: int, batch: int, heads: int, tokens: int, head_dim: int,
             dist: str = "iid", outlier_frac: float = 0.0,
             outlier_scale: float = 8.0):
    """Return (K, V) as float16 arrays of shape [B, H, T, d]."""
    rng = np.random.default_rng(seed)
    shape = (batch, heads, tokens, head_dim)
    if dist == "iid":
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "channel":
        sk = channel_scales(rng, heads, head_dim, outlier_frac, outlier_scale)
        sv = channel_scales(rng, heads, head_dim, outlier_frac, outlier_scale)
        k = rng.standard_normal(shape, dtype=np.float32) * sk[None, :, None, :]
        v = rng.standard_normal(shape, dtype=np.float32) * sv[None, :, None, :]
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return k.astype(np.float16), v.astype(np.float16)


def q_numpy(seed: int, batch: int, q_heads: int, head_dim: int) -> np.ndarray:
    """Queries, float16 [B, Hq, d], N(0, 1)."""
    rng = np.random.default_rng(seed + 0x5151)
    return rng.standard_normal((batch, q_heads, head_dim),
                               dtype=np.float32).astype(np.float16)


def kv_torch(seed: int, batch: int, heads: int, tokens: int, head_dim: int,
             dist: str = "iid", outlier_frac: float = 0.0,
             outlier_scale: float = 8.0, device="cuda"):
    """Device-side (K, V) float16 [B, H, T, d] for sizes too large for numpy.

    The per-channel scales come from the numpy generator above (they are
    tiny); the bulk normals come from a seeded ``torch.Generator`` on the
    device, drawn one (batch, head) slab at a time to bound temporaries.
    """
    import torch
    rng = np.random.default_rng(seed)
    if dist == "channel":
        sk = channel_scales(rng, heads, head_dim, outlier_frac, outlier_scale)
        sv = channel_scales(rng, heads, head_dim, outlier_frac, outlier_scale)
    elif dist == "iid":
        sk = np.ones((heads, head_dim), np.float32)
        sv = np.ones((heads, head_dim), np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for s in (sk, sv):
        st = torch.from_numpy(s).to(device)
        t = torch.empty((batch, heads, tokens, head_dim), dtype=torch.float16,
                        device=device)
        for b in range(batch):
            for h in range(heads):
                x = torch.randn((tokens, head_dim), generator=g,
                                dtype=torch.float32, device=device)
                t[b, h] = (x * st[h]).to(torch.float16)
        out.append(t)
    return out[0], out[1]


def q_torch(seed: int, batch: int, q_heads: int, head_dim: int,
            device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed + 0x5151)
    return torch.randn((batch, q_heads, head_dim), generator=g,
                       dtype=torch.float32, device=device).to(torch.float16)


def peak_keys_torch(k, q, start: int, period: int = 512, count: int = 4, gain: float = 9.0):
    """Heavy-hitter keys for a peaked softmax: in the K rows k [B, H, n, d]
    (positions start .. start + n - 1), the positions t with t mod period <
    count are replaced by gain times the mean of the KV head's query group
    (q [B, Hq, d]); every other row is left as drawn.  With N(0, 1) queries
    those positions' logits lie far above the rest."""
    import torch
    B, H, n, d = k.shape
    G = q.shape[1] // H
    qbar = q.float().reshape(B, H, G, d).mean(dim=2)                   # [B, H, d]
    t = torch.arange(start, start + n, device=k.device)
    hot = (t % period) < count
    if bool(hot.any()):
        k[:, :, hot] = (gain * qbar)[:, :, None, :].to(k.dtype)
    return k


# The five workload shapes.  ``dist`` / ``outliers`` give the input recipe;
# ``append`` is the number of tokens appended per sequence inside one step
# ("prefill" = the chunk size of the prefill quantize-append).
CONFIGS = {
    "c1_small": dict(batch=1, kv_heads=2, q_heads=4, head_dim=64, tokens=256,
                     layers=1, k_mode="packed", k_bits=3, v_mode="packed",
                     v_bits=4, dist="iid", outlier_frac=0.0, append=256),
    "c2_sym4_4k": dict(batch=1, kv_heads=8, q_heads=32, head_dim=128,
                       tokens=4096, layers=36, k_mode="packed", k_bits=4,
                       v_mode="packed", v_bits=4, dist="channel",
                       outlier_frac=0.01, append=0),
    "c3_asym_16k": dict(batch=8, kv_heads=8, q_heads=32, head_dim=128,
                        tokens=16384, layers=36, k_mode="fp16", k_bits=0,
                        v_mode="packed", v_bits=4, dist="channel",
                        outlier_frac=0.01, append=1),
    "c4_tq35_32k": dict(batch=4, kv_heads=8, q_heads=32, head_dim=128,
                        tokens=32768, layers=36, k_mode="packed", k_bits=3,
                        v_mode="packed", v_bits=4, dist="channel",
                        outlier_frac=0.01, append=0, prefill=8192),
    "c5_delegated_64k": dict(batch=16, kv_heads=4, q_heads=32, head_dim=128,
                             tokens=65536, layers=48, k_mode="fp16", k_bits=0,
                             v_mode="delegated", v_bits=4, hot=256,
                             dist="channel", outlier_frac=0.0, append=0),
}
