"""Seeded BF16 query/key/value tensors.

Values are N(0,1) in FP32, K gets 4 fixed outlier channels per (layer,
kv-head) scaled by 20 (the outlier-channel situation that the Hadamard
rotation of keys addresses, paper.rainbus.top summary, "分组仿射 KV 量化"),
then everything is rounded to BF16.  Keys and queries are taken to be
post-RoPE already.  The streams are torch generators keyed by
(seed, layer) so that the same call gives the same tensors on the CPU every
time, and large workloads can be drawn directly in device memory.
"""
from __future__ import annotations

import numpy as np
import torch

N_OUTLIERS = 4
OUTLIER_SCALE = 20.0


def outlier_channels(seed: int, layer: int, Hkv: int, head_dim: int = 128) -> np.ndarray:
    """int64 [Hkv][4]: outlier channel ids, drawn without replacement."""
    rng = np.random.default_rng([seed, layer, 0x0C7])
    return np.stack([rng.choice(head_dim, N_OUTLIERS, replace=False) for _ in range(Hkv)])


def _key(seed: int, layer: int, stream: int) -> int:
    return (seed * 1_000_003 + layer * 7919 + stream) & 0x7FFF_FFFF_FFFF


def draw_values(seed: int, layer: int, n_tokens: int, B: int, Hq: int, Hkv: int,
                device="cpu", head_dim: int = 128):
    """Return (k, v, q) as BF16 tensors:
    k, v: [n_tokens][Hkv][head_dim] (token-major, all sequences back to back),
    q:    [B][Hq][head_dim]."""
    out = []
    for stream, shape in enumerate(((n_tokens, Hkv, head_dim), (n_tokens, Hkv, head_dim),
                                    (B, Hq, head_dim))):
        g = torch.Generator(device=device)
        g.manual_seed(_key(seed, layer, stream))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if stream == 0:
            scale = torch.ones((Hkv, head_dim), dtype=torch.float32)
            ch = outlier_channels(seed, layer, Hkv, head_dim)
            for h in range(Hkv):
                scale[h, ch[h]] = OUTLIER_SCALE
            x.mul_(scale.to(device))
        out.append(x.to(torch.bfloat16))
    return tuple(out)
