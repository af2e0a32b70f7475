"""GPU parity of the KV8-everywhere variant (the INT8 point of the pages'
quantization-target comparison) against the oracle's KV8 path on the same
seeded inputs: pool bytes, query codes and int32 QK bit-exact, out within
2e-3 and lse within 1e-4."""
import math

import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from synth import draw_values, make_workload
from tests.gpu_util import SCALE, bf, i32
from tests.wl import bf16_bits, host_inputs

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4
EDGE = [1, 2, 15, 16, 17, 31, 32, 33, 143, 144, 145, 300, 1000]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _oracle_kv8(wl, hi):
    cache = oracle.Kv8Cache(wl.num_pages, wl.Hkv)
    k, v, cu = hi.prefix(wl.ctx - 1)
    oracle.kv8_prefill(cache, k, v, cu, np.zeros(wl.B, np.int32), wl.page_table)
    ka, va = hi.at(wl.ctx - 1)
    oracle.kv8_append(cache, ka, va, (wl.ctx - 1).astype(np.int32), wl.page_table)
    return cache


def _gpu_kv8(wl, hi, dev, use_prefill=True):
    cache = kv4.Kv8Cache.zeros(wl.num_pages, wl.Hkv, dev)
    table = i32(wl.page_table, dev)
    lead = wl.ctx - 1
    if use_prefill:
        k, v, cu = hi.prefix(lead)
        if len(k):
            kv4.kv8_prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev),
                                     table, int(max(1, lead.max())))
    else:
        for p in range(int(lead.max())):
            rows = np.nonzero(lead > p)[0]
            if len(rows):
                ka, va = hi.at(np.full(wl.B, p))
                kv4.kv8_append(cache, bf(ka[rows], dev), bf(va[rows], dev), i32(np.full(len(rows), p), dev),
                               i32(wl.page_table[rows], dev))
    ka, va = hi.at(wl.ctx - 1)
    kv4.kv8_append(cache, bf(ka, dev), bf(va, dev), i32(wl.ctx - 1, dev), table)
    return cache, table


def _check(wl, hi, dev):
    ref = _oracle_kv8(wl, hi)
    cache, table = _gpu_kv8(wl, hi, dev)
    q, ctx = bf(hi.q, dev), i32(wl.ctx, dev)
    out, lse = kv4.kv8_decode_attention(cache, q, ctx, table, wl.max_ctx, SCALE)
    out_d, lse_d, dbg = kv4.kv8_decode_attention_debug(cache, q, ctx, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pages.cpu().numpy(), ref.pages), "KV8 pool bytes differ"
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    r_out, r_lse, r_dbg = oracle.kv8_decode(ref, hi.q, wl.ctx.astype(np.int32), wl.page_table, wl.Hq,
                                            SCALE, debug=True)
    for key in ("qcodes", "qsum", "qk"):
        got = dbg[key].cpu().numpy()
        bad = np.argwhere(got != r_dbg[key])
        assert len(bad) == 0, f"{key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)
    return err, lerr


@pytest.mark.parametrize("name,kw", [("edges_8_2", dict(ctx=EDGE, Hq=8, Hkv=2, seed=51)),
                                     ("edges_4_1", dict(ctx=EDGE[::-1], Hq=4, Hkv=1, seed=52))])
def test_kv8_parity_edges(name, kw):
    _say(f"[kv8] {name}")
    wl = make_workload(0, **kw)
    err, lerr = _check(wl, host_inputs(wl), torch.device("cuda"))
    _say(f"[kv8] {name}: out {err:.2e} lse {lerr:.2e}")


def test_kv8_appends_equal_prefill():
    _say("[kv8] appends == prefill")
    wl = make_workload(0, ctx=EDGE[::2], Hq=4, Hkv=1, seed=53)
    hi = host_inputs(wl)
    dev = torch.device("cuda")
    a, _ = _gpu_kv8(wl, hi, dev, use_prefill=False)
    b, _ = _gpu_kv8(wl, hi, dev, use_prefill=True)
    torch.cuda.synchronize()
    assert torch.equal(a.pages, b.pages)


def test_kv8_short_workload():
    _say("[kv8] short workload B=64")
    wl = make_workload(1)
    err, lerr = _check(wl, host_inputs(wl), torch.device("cuda"))
    _say(f"[kv8] short: out {err:.2e} lse {lerr:.2e}")


def test_kv8_fullsize_sampled():
    """The 256-sequence benchmark workload decoded on the GPU in one launch;
    a sample of sequences rebuilt and decoded by the oracle."""
    dev = torch.device("cuda")
    wl = make_workload(4)
    _say(f"[kv8] full size B={wl.B} mean ctx {wl.ctx.mean():.0f}")
    n_tok = int(wl.ctx.sum())
    k, v, q = draw_values(wl.seed, 0, n_tok, wl.B, wl.Hq, wl.Hkv, device=dev)
    off = np.zeros(wl.B + 1, np.int64)
    off[1:] = np.cumsum(wl.ctx)
    lead = wl.ctx - 1
    rows = torch.from_numpy(np.concatenate([np.arange(off[b], off[b] + lead[b]) for b in range(wl.B)])).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)).to(dev)
    table = torch.from_numpy(wl.page_table).to(dev)
    cache = kv4.Kv8Cache.zeros(wl.num_pages, wl.Hkv, dev)
    kv4.kv8_prefill_quantize(cache, k[rows].contiguous(), v[rows].contiguous(), cu,
                             torch.zeros(wl.B, dtype=torch.int32, device=dev), table, int(lead.max()))
    last = torch.from_numpy(off[:-1] + lead).to(dev)
    kv4.kv8_append(cache, k[last].contiguous(), v[last].contiguous(), i32(wl.ctx - 1, dev), table)
    ctx = i32(wl.ctx, dev)
    out, lse = kv4.kv8_decode_attention(cache, q, ctx, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    order = np.argsort(wl.ctx, kind="stable")
    sample = np.unique([order[0], order[len(order) // 2], order[-1], 7])
    _say(f"[kv8] oracle on sequences {sample.tolist()} (ctx {wl.ctx[sample].tolist()})")
    ctx_s = wl.ctx[sample]
    need = (ctx_s + 15) // 16
    rtable = np.zeros((len(sample), int(need.max())), np.int32)
    o = 0
    for i, n in enumerate(need):
        rtable[i, :n] = np.arange(o, o + n)
        o += n
    ref = oracle.Kv8Cache(int(need.sum()), wl.Hkv)
    allrows = np.concatenate([np.arange(off[b], off[b] + wl.ctx[b]) for b in sample])
    kh = bf16_bits(k[torch.from_numpy(allrows).to(dev)])
    vh = bf16_bits(v[torch.from_numpy(allrows).to(dev)])
    cu_s = np.concatenate([[0], np.cumsum(ctx_s)]).astype(np.int32)
    oracle.kv8_prefill(ref, kh, vh, cu_s, np.zeros(len(sample), np.int32), rtable)
    r_out, r_lse, _ = oracle.kv8_decode(ref, bf16_bits(q[torch.from_numpy(sample).to(dev)]),
                                        ctx_s.astype(np.int32), rtable, wl.Hq, SCALE)
    sel = torch.from_numpy(sample).to(dev)
    err = float(np.abs(out[sel].cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse[sel].cpu().numpy() - r_lse).max())
    _say(f"[kv8] full size: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
