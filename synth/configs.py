"""The five synthetic decode workloads (shapes, lengths, page tables, slots).

Every workload is GQA decode with head_dim 128 and 16-position pages; the
KV4-RL pages fix sink s=16 and recent window w=128 (paper.rainbus.top summary,
"核心方法"), the default protection budget of the cache descriptor (other
budgets are descriptor fields too).

  tiny     B=4,   Hq/Hkv=4/1,  ctx {100,144,400,700}, 128-page pool (width 64)
  short    B=64,  32/8, prompt U[128,512] + length-biased lognormal(1450, 1087.5)
  async    B=512, 32/8, prompt U[128,512] + length-biased lognormal(4000, 3000)
  longtail B=128, 32/8, ctx uniform on [12000, 16896], zero-slack pool
  qwen8b   B=256, 32/8, prompt U[128,512] + length-biased lognormal(3000, 2250),
           36 layers; plus a 8 x 16384-token re-prefill

Readings: a context length counts the token appended this step; where a
standard deviation is not given (short, qwen8b) the coefficient of variation
0.75 of the async workload is borrowed; the tiny workload's "64-page pool"
cannot hold sum(ceil(L/16)) = 85 pages, so its page table is 64 entries wide
and its physical pool has 128 pages.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .lengths import sample_contexts

PAGE = 16
HEAD_DIM = 128


@dataclass
class Workload:
    name: str
    index: int
    B: int
    Hq: int
    Hkv: int
    ctx: np.ndarray            # int64 [B], includes this step's token
    page_table: np.ndarray     # int32 [B][pt_stride], physical page ids
    num_pages: int
    slots: np.ndarray          # int32 [B]
    max_slots: int
    layers: int = 1
    append_step: bool = True   # cache holds ctx-1 positions, then one append
    seed: int = 0
    prefill_nseq: int = 0
    prefill_len: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def max_ctx(self) -> int:
        return int(self.ctx.max())

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


def pages_needed(ctx: np.ndarray) -> np.ndarray:
    return (ctx + PAGE - 1) // PAGE


def build_page_table(rng: np.random.Generator, ctx: np.ndarray, num_pages: int,
                     pt_stride: int) -> np.ndarray:
    """Give every sequence ceil(L/16) distinct physical pages, taken in order
    from a seeded random permutation of the pool (a fragmented table).
    Unused entries hold page 0 so that no entry is ever out of the pool."""
    need = pages_needed(ctx)
    assert int(need.sum()) <= num_pages and int(need.max()) <= pt_stride
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.zeros((len(ctx), pt_stride), dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table


def _lengths(index: int, rng: np.random.Generator, B: int) -> np.ndarray:
    if index == 0:
        return np.array([100, 144, 400, 700], dtype=np.int64)
    if index == 1:
        return sample_contexts(rng, B, 1450.0, 0.75 * 1450.0)
    if index == 2:
        return sample_contexts(rng, B, 4000.0, 3000.0)
    if index == 3:
        return rng.integers(12000, 16896 + 1, size=B).astype(np.int64)
    if index == 4:
        return sample_contexts(rng, B, 3000.0, 0.75 * 3000.0)
    raise ValueError(index)


CONFIGS = {
    0: dict(name="tiny", B=4, Hq=4, Hkv=1, layers=1, append_step=True),
    1: dict(name="short", B=64, Hq=32, Hkv=8, layers=1, append_step=True),
    2: dict(name="async", B=512, Hq=32, Hkv=8, layers=1, append_step=False),
    3: dict(name="longtail", B=128, Hq=32, Hkv=8, layers=1, append_step=False),
    4: dict(name="qwen8b", B=256, Hq=32, Hkv=8, layers=36, append_step=True,
            prefill_nseq=8, prefill_len=16384),
}


def make_workload(index: int, seed: int | None = None, ctx=None, B=None,
                  Hq=None, Hkv=None, pool_slack: int = 0) -> Workload:
    """Build workload `index` (0..4).  `ctx`/`B`/`Hq`/`Hkv` override the
    configured values (used by property tests); `seed` defaults to the index."""
    cfg = dict(CONFIGS[index])
    seed = index if seed is None else seed
    rng = np.random.default_rng(seed)
    B = cfg["B"] if B is None else B
    if ctx is None:
        ctx = _lengths(index, rng, B)
    ctx = np.asarray(ctx, dtype=np.int64)
    B = len(ctx)
    Hq = cfg["Hq"] if Hq is None else Hq
    Hkv = cfg["Hkv"] if Hkv is None else Hkv
    need = pages_needed(ctx)
    if index == 0 and pool_slack == 0 and len(ctx) == 4:
        num_pages, pt_stride = 128, 64
    else:
        num_pages = int(need.sum()) + pool_slack
        pt_stride = int(need.max())
    table = build_page_table(rng, ctx, num_pages, pt_stride)
    slots = np.arange(B, dtype=np.int32)
    return Workload(name=cfg["name"], index=index, B=B, Hq=Hq, Hkv=Hkv, ctx=ctx,
                    page_table=table, num_pages=num_pages, slots=slots,
                    max_slots=B, layers=cfg["layers"],
                    append_step=cfg["append_step"], seed=seed,
                    prefill_nseq=cfg.get("prefill_nseq", 0),
                    prefill_len=cfg.get("prefill_len", 0))
