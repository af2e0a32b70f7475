"""Helpers for GPU tests: move synthetic host inputs to the device and build a
cache there through the library (re-prefill of the leading positions, then
this step's append)."""
from __future__ import annotations

import math

import numpy as np
import torch

import int8_mixed_precision_kv4_amd as kv4

SCALE = 1.0 / math.sqrt(128)


def bf(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


class GpuCase:
    """Device-side state of one workload layer."""

    def __init__(self, wl, hi, dev="cuda", use_prefill=True, sink=kv4.SINK, window=kv4.WINDOW):
        self.wl, self.hi, self.dev = wl, hi, torch.device(dev)
        self.cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, self.dev, sink, window)
        self.table = i32(wl.page_table, self.dev)
        self.slots = i32(wl.slots, self.dev)
        self.ctx = i32(wl.ctx, self.dev)
        self.q = bf(hi.q, self.dev)
        lead = wl.ctx - 1 if wl.append_step else wl.ctx
        if use_prefill:
            k, v, cu = hi.prefix(lead)
            if len(k):
                kv4.prefill_quantize(self.cache, bf(k, self.dev), bf(v, self.dev), i32(cu, self.dev),
                                     i32(np.zeros(wl.B), self.dev), self.slots, self.table,
                                     int(max(1, lead.max())))
        else:
            for p in range(int(lead.max())):
                rows = np.nonzero(lead > p)[0]
                ka, va = hi.at(np.full(wl.B, p))
                self._append_rows(rows, ka, va, p)
        if wl.append_step:
            ka, va = hi.at(wl.ctx - 1)
            kv4.append(self.cache, bf(ka, self.dev), bf(va, self.dev), i32(wl.ctx - 1, self.dev),
                       self.slots, self.table)

    def _append_rows(self, rows, ka, va, p):
        if len(rows) == 0:
            return
        kv4.append(self.cache, bf(ka[rows], self.dev), bf(va[rows], self.dev),
                   i32(np.full(len(rows), p), self.dev), i32(self.wl.slots[rows], self.dev),
                   i32(self.wl.page_table[rows], self.dev))

    def decode(self, debug=False):
        if debug:
            return kv4.decode_attention_debug(self.cache, self.q, self.ctx, self.slots, self.table,
                                              self.wl.max_ctx, SCALE)
        return kv4.decode_attention(self.cache, self.q, self.ctx, self.slots, self.table,
                                    self.wl.max_ctx, SCALE)
