"""Test helpers: turn a synthetic workload into host arrays and an oracle cache."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle
from synth import draw_values, make_workload  # noqa: F401  (re-exported for tests)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@dataclass
class HostInputs:
    k: np.ndarray        # uint16 [sum ctx][Hkv][128]  all positions of all sequences
    v: np.ndarray
    q: np.ndarray        # uint16 [B][Hq][128]
    offsets: np.ndarray  # int64 [B+1] row offset of each sequence in k/v

    def prefix(self, lengths):
        """Packed rows for positions [0, lengths[b]) of every sequence."""
        rows = np.concatenate([np.arange(self.offsets[b], self.offsets[b] + n)
                               for b, n in enumerate(lengths)]) if len(lengths) else np.zeros(0, int)
        cu = np.zeros(len(lengths) + 1, np.int32)
        cu[1:] = np.cumsum(lengths)
        return self.k[rows], self.v[rows], cu

    def at(self, positions):
        """Rows at position positions[b] of every sequence: [B][Hkv][128]."""
        rows = self.offsets[:-1] + np.asarray(positions)
        return self.k[rows], self.v[rows]


def host_inputs(wl, layer: int = 0) -> HostInputs:
    n = int(wl.ctx.sum())
    k, v, q = draw_values(wl.seed, layer, n, wl.B, wl.Hq, wl.Hkv, device="cpu")
    off = np.zeros(wl.B + 1, np.int64)
    off[1:] = np.cumsum(wl.ctx)
    return HostInputs(bf16_bits(k), bf16_bits(v), bf16_bits(q), off)


def oracle_cache(wl, hi: HostInputs, nthreads=None, sink=oracle.SINK,
                 window=oracle.WINDOW) -> oracle.Cache:
    """Cache state right before attention: positions [0, ctx-1) by re-prefill,
    then this step's token appended (or all ctx positions by re-prefill for
    decode-only workloads); sink / window: the protection budget."""
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    lead = wl.ctx - 1 if wl.append_step else wl.ctx
    k, v, cu = hi.prefix(lead)
    oracle.prefill(cache, k, v, cu, np.zeros(wl.B, np.int32), wl.slots, wl.page_table, nthreads)
    if wl.append_step:
        ka, va = hi.at(wl.ctx - 1)
        oracle.append(cache, ka, va, (wl.ctx - 1).astype(np.int32), wl.slots, wl.page_table)
    return cache
