"""GPU parity of the MXFP4 variant (OCP MXFP4 main region, the rest of KV4-RL
unchanged) against the oracle's MXFP4 path on the same seeded inputs: page
blocks (codes and E8M0 scales) and side rows bit-exact, out within 2e-3 and
lse within 1e-4."""
import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from synth import make_workload
from tests.gpu_util import SCALE, bf, i32
from tests.test_gpu_parity import assert_cache_equal
from tests.wl import host_inputs

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4
EDGE = [1, 2, 15, 16, 17, 143, 144, 145, 146, 159, 160, 161, 177, 300, 1000]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


class _Case:
    def __init__(self, wl, hi, sink, window, dev, use_prefill=True):
        self.wl, self.hi = wl, hi
        self.cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, sink, window)
        self.table, self.slots = i32(wl.page_table, dev), i32(wl.slots, dev)
        lead = wl.ctx - 1
        if use_prefill:
            k, v, cu = hi.prefix(lead)
            if len(k):
                kv4.mx_prefill_quantize(self.cache, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev),
                                        self.slots, self.table, int(max(1, lead.max())))
        else:
            for p in range(int(lead.max())):
                rows = np.nonzero(lead > p)[0]
                if len(rows):
                    ka, va = hi.at(np.full(wl.B, p))
                    kv4.mx_append(self.cache, bf(ka[rows], dev), bf(va[rows], dev), i32(np.full(len(rows), p), dev),
                                  i32(wl.slots[rows], dev), i32(wl.page_table[rows], dev))
        ka, va = hi.at(wl.ctx - 1)
        kv4.mx_append(self.cache, bf(ka, dev), bf(va, dev), i32(wl.ctx - 1, dev), self.slots, self.table)


def _oracle_mx(wl, hi, sink, window):
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    k, v, cu = hi.prefix(wl.ctx - 1)
    oracle.mx_prefill(cache, k, v, cu, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    ka, va = hi.at(wl.ctx - 1)
    oracle.mx_append(cache, ka, va, (wl.ctx - 1).astype(np.int32), wl.slots, wl.page_table)
    return cache


@pytest.mark.parametrize("name,kw,s,w", [
    ("edges_8_2", dict(ctx=EDGE, Hq=8, Hkv=2, seed=71), 16, 128),
    ("edges_unprotected", dict(ctx=EDGE[::-1], Hq=4, Hkv=1, seed=72), 0, 0),
    ("short", dict(), 16, 128),
])
def test_mx_parity(name, kw, s, w):
    _say(f"[mx] {name} s={s} w={w}")
    dev = torch.device("cuda")
    wl = make_workload(1 if name == "short" else 0, **kw)
    hi = host_inputs(wl)
    ref = _oracle_mx(wl, hi, s, w)
    case = _Case(wl, hi, s, w, dev)
    q, ctx = bf(hi.q, dev), i32(wl.ctx, dev)
    out, lse = kv4.mx_decode_attention(case.cache, q, ctx, case.slots, case.table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    r_out, r_lse = oracle.mx_decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[mx] {name}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)


def test_mx_appends_equal_prefill():
    _say("[mx] appends == prefill")
    dev = torch.device("cuda")
    wl = make_workload(0, ctx=EDGE[::2], Hq=4, Hkv=1, seed=73)
    hi = host_inputs(wl)
    a = _Case(wl, hi, 16, 128, dev, use_prefill=False)
    b = _Case(wl, hi, 16, 128, dev, use_prefill=True)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.pages, b.cache.pages)
    assert torch.equal(a.cache.side_codes, b.cache.side_codes)


def test_mx_fullsize_sampled():
    """The 256-sequence benchmark workload written and decoded in the MXFP4
    variant on the GPU in the benchmark's launch configuration; a sample of
    sequences rebuilt (prefill of the prefix, append of the last token) and
    decoded by the oracle."""
    from synth import draw_values
    from tests.wl import bf16_bits
    dev = torch.device("cuda")
    wl = make_workload(4)
    _say(f"[mx] full size B={wl.B} mean ctx {wl.ctx.mean():.0f}")
    n_tok = int(wl.ctx.sum())
    k, v, q = draw_values(wl.seed, 0, n_tok, wl.B, wl.Hq, wl.Hkv, device=dev)
    off = np.zeros(wl.B + 1, np.int64)
    off[1:] = np.cumsum(wl.ctx)
    lead = wl.ctx - 1
    rows = torch.from_numpy(np.concatenate([np.arange(off[b], off[b] + lead[b]) for b in range(wl.B)])).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)).to(dev)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev)
    kv4.mx_prefill_quantize(cache, k[rows].contiguous(), v[rows].contiguous(), cu,
                            torch.zeros(wl.B, dtype=torch.int32, device=dev), slots, table, int(lead.max()))
    last = torch.from_numpy(off[:-1] + lead).to(dev)
    kv4.mx_append(cache, k[last].contiguous(), v[last].contiguous(), i32(lead, dev), slots, table)
    out, lse = kv4.mx_decode_attention(cache, q, i32(wl.ctx, dev), slots, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    order = np.argsort(wl.ctx, kind="stable")
    sample = np.unique([order[0], order[len(order) // 2], order[-1], 11])
    _say(f"[mx] oracle on sequences {sample.tolist()} (ctx {wl.ctx[sample].tolist()})")
    ctx_s = wl.ctx[sample]
    need = (ctx_s + 15) // 16
    rtable = np.zeros((len(sample), int(need.max())), np.int32)
    o = 0
    for i, n in enumerate(need):
        rtable[i, :n] = np.arange(o, o + n)
        o += n
    ref = oracle.Cache(int(need.sum()), wl.Hkv, len(sample))
    lead_s = ctx_s - 1
    prow = np.concatenate([np.arange(off[b], off[b] + lead[b]) for b in sample])
    cu_s = np.concatenate([[0], np.cumsum(lead_s)]).astype(np.int32)
    oracle.mx_prefill(ref, bf16_bits(k[torch.from_numpy(prow).to(dev)]), bf16_bits(v[torch.from_numpy(prow).to(dev)]),
                      cu_s, np.zeros(len(sample), np.int32), np.arange(len(sample), dtype=np.int32), rtable)
    lrow = torch.from_numpy(off[sample] + lead_s).to(dev)
    oracle.mx_append(ref, bf16_bits(k[lrow]), bf16_bits(v[lrow]), lead_s.astype(np.int32),
                     np.arange(len(sample), dtype=np.int32), rtable)
    r_out, r_lse = oracle.mx_decode(ref, bf16_bits(q[torch.from_numpy(sample).to(dev)]), ctx_s.astype(np.int32),
                                    np.arange(len(sample), dtype=np.int32), rtable, wl.Hq, SCALE)
    sel = torch.from_numpy(sample).to(dev)
    err = float(np.abs(out[sel].cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse[sel].cpu().numpy() - r_lse).max())
    _say(f"[mx] full size: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)
