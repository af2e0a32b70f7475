"""GPU parity of the re-prefill (chunked-prefill) attention against the
oracle on the same seeded inputs: query codes, int32 QK, P-operand codes and
int32 PV accumulators bit-exact, out within 2e-3 and lse within 1e-4; a
one-token chunk reproduces the decode step (the integer intermediates bit for
bit, out and lse up to the FP32 order of the tile merges, which the method
leaves free)."""
import math

import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from synth import make_workload
from tests.gpu_util import SCALE, bf, i32
from tests.wl import host_inputs

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _queries(T, Hq, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, 128)).astype(np.float32)
    return torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _setup(ctx, n, Hq, Hkv, seed, sink=16, window=128, k_scale_every=0):
    """Caches (GPU and oracle) holding [0, ctx) of every sequence, written by
    re-prefill; chunk = the last n[s] positions.  k_scale_every = j > 0: the
    keys of every j-th row (all sequences back to back) times 1000."""
    dev = torch.device("cuda")
    wl = make_workload(0, ctx=ctx, Hq=Hq, Hkv=Hkv, seed=seed)
    hi = host_inputs(wl)
    if k_scale_every:
        kf = torch.from_numpy(hi.k.view(np.int16)).view(torch.bfloat16).float()
        kf[::k_scale_every] *= 1000.0
        hi.k = kf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    k, v, cu_all = hi.prefix(wl.ctx)
    ref = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    oracle.prefill(ref, k, v, cu_all, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, sink, window)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu_all, dev), i32(np.zeros(wl.B), dev), slots, table,
                         int(wl.ctx.max()))
    n = np.asarray(n, np.int32)
    start = (wl.ctx - n).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = _queries(int(cu[-1]), Hq, seed + 1)
    return dev, wl, ref, cache, table, slots, start, cu, q


@pytest.mark.parametrize("name,ctx,n,Hq,Hkv,sw", [
    ("mixed_8_2", [230, 60, 17, 400], [40, 23, 17, 1], 8, 2, (16, 128)),
    ("long_chunk_4_1", [300, 1000], [300, 200], 4, 1, (16, 128)),
    ("unprotected", [150, 64], [50, 64], 4, 1, (0, 0)),
])
def test_prefill_attention_parity(name, ctx, n, Hq, Hkv, sw):
    _say(f"[chunk] {name}")
    dev, wl, ref, cache, table, slots, start, cu, q = _setup(ctx, n, Hq, Hkv, 91, *sw)
    qd = bf(q, dev)
    max_ctx = int(wl.ctx.max())
    out, lse = kv4.prefill_attention(cache, qd, i32(cu, dev), i32(start, dev), slots, table, max_ctx, SCALE)
    out_d, lse_d, dbg = kv4.prefill_attention_debug(cache, qd, i32(cu, dev), i32(start, dev), slots, table,
                                                    max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, wl.slots, wl.page_table, Hq, SCALE,
                                                   debug=True)
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        got = dbg[key].cpu().numpy()
        bad = np.argwhere(got != r_dbg[key])
        assert len(bad) == 0, f"{key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[chunk] {name}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)


def test_one_token_chunks_equal_decode():
    _say("[chunk] one-token chunks == decode")
    dev, wl, ref, cache, table, slots, start, cu, q = _setup([1, 17, 145, 300], [1, 1, 1, 1], 8, 2, 93)
    qd = bf(q, dev)
    max_ctx = int(wl.ctx.max())
    out, lse, dbg = kv4.prefill_attention_debug(cache, qd, i32(cu, dev), i32(start, dev), slots, table,
                                                max_ctx, SCALE)
    o2, l2, d2 = kv4.decode_attention_debug(cache, qd, i32(wl.ctx, dev), slots, table, max_ctx, SCALE)
    torch.cuda.synchronize()
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        assert torch.equal(dbg[key], d2[key]), key
    assert float((out - o2).abs().max()) <= 1e-5 and float((lse - l2).abs().max()) <= 1e-6


def test_chunk_blocks_and_budgets():
    """Chunks of every length mod 8 (partial token blocks), several chunks per
    call, with the default, an all-sink and an unprotected budget."""
    _say("[chunk] block tails and budgets")
    for sw in ((16, 128), (144, 0), (0, 0)):
        dev, wl, ref, cache, table, slots, start, cu, q = _setup(
            [9, 170, 300, 64, 500, 33, 257, 18], [9, 65, 3, 64, 130, 7, 100, 2], 4, 1, 95, *sw)
        qd = bf(q, dev)
        max_ctx = int(wl.ctx.max())
        out, lse, dbg = kv4.prefill_attention_debug(cache, qd, i32(cu, dev), i32(start, dev), slots, table,
                                                    max_ctx, SCALE)
        torch.cuda.synchronize()
        r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, wl.slots, wl.page_table, 4, SCALE,
                                                       debug=True)
        for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
            got = dbg[key].cpu().numpy()
            assert np.array_equal(got, r_dbg[key]), (sw, key, np.argwhere(got != r_dbg[key])[:4].tolist())
        err = float(np.abs(out.cpu().numpy() - r_out).max())
        lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
        _say(f"[chunk] budget {sw}: out {err:.2e} lse {lerr:.2e}")
        assert err <= OUT_TOL and lerr <= LSE_TOL, (sw, err, lerr)


def test_wide_logit_spread_in_whole_pairs():
    """Keys of every 5th row scaled by 1000: in most tiles one logit then lies
    hundreds (base 2) above or below the others, so the pairs every row sees
    whole take exp2s with its select below -125 (weights exactly 0), not the
    form without it, which needs every logit of the pair within 125 of its
    tile's max.  Integer intermediates bit-exact, out to the bar, lse to the
    bar relative to max(1, |lse|)."""
    _say("[chunk] wide logit spread")
    dev, wl, ref, cache, table, slots, start, cu, q = _setup([700, 520], [96, 64], 8, 2, 97, k_scale_every=5)
    qd = bf(q, dev)
    max_ctx = int(wl.ctx.max())
    out, lse = kv4.prefill_attention(cache, qd, i32(cu, dev), i32(start, dev), slots, table, max_ctx, SCALE)
    out_d, lse_d, dbg = kv4.prefill_attention_debug(cache, qd, i32(cu, dev), i32(start, dev), slots, table,
                                                    max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, wl.slots, wl.page_table, 8, SCALE,
                                                   debug=True)
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        got = dbg[key].cpu().numpy()
        bad = np.argwhere(got != r_dbg[key])
        assert len(bad) == 0, f"{key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    # the case is the one meant: many main-region codes are 0 next to a 127
    codes = r_dbg["pcode"][:, :, 16:wl.ctx.min() - 128]
    assert (codes == 0).mean() > 0.5 and (codes == 127).any()
    # lse is near ln 2 times the largest logit (hundreds here): FP32 resolves
    # it to a few 1e-5 relative whatever the order of the merges, so its bar
    # scales with it above 1
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float((np.abs(lse.cpu().numpy() - r_lse) / np.maximum(1.0, np.abs(r_lse))).max())
    _say(f"[chunk] wide logit spread: out {err:.2e} lse {lerr:.2e} relative (|lse| up to "
         f"{float(np.abs(r_lse).max()):.0f})")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)


def test_nan_key_scale_in_whole_pairs():
    """A NaN key scale (FP16 metadata bits 0x7E00, outside what the quantizer
    writes) at three main-region positions of sequence 0 in both caches: their
    logits are NaN, which the tile max leaves out and exp2s maps to weight 0.
    In the pairs every row sees whole, such a pair must take the selecting
    exp2s: the test on the smallest logit of a tile propagates NaN.  Integer
    intermediates bit-exact, out and lse finite and to the bar."""
    _say("[chunk] NaN key scales")
    dev, wl, ref, cache, table, slots, start, cu, q = _setup([700, 300], [96, 40], 8, 2, 99)
    for pos in (40, 77, 200):
        page, off = int(wl.page_table[0, pos // 16]), 2048 + 4 * (pos % 16)
        ref.pages[page, :, off], ref.pages[page, :, off + 1] = 0x00, 0x7E
        cache.pages[page, :, off], cache.pages[page, :, off + 1] = 0x00, 0x7E
    qd = bf(q, dev)
    max_ctx = int(wl.ctx.max())
    out, lse = kv4.prefill_attention(cache, qd, i32(cu, dev), i32(start, dev), slots, table, max_ctx, SCALE)
    out_d, lse_d, dbg = kv4.prefill_attention_debug(cache, qd, i32(cu, dev), i32(start, dev), slots, table,
                                                    max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, wl.slots, wl.page_table, 8, SCALE,
                                                   debug=True)
    assert np.isfinite(r_out).all() and np.isfinite(r_lse).all()
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        got = dbg[key].cpu().numpy()
        bad = np.argwhere(got != r_dbg[key])
        assert len(bad) == 0, f"{key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    assert (r_dbg["pcode"][:int(cu[1]), :, [40, 77, 200]] == 0).all()
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[chunk] NaN key scales: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)


def test_benchmark_reprefill_sampled():
    """The benchmark's re-prefill (8 chunks of 16,384 tokens, 32/8 heads, the
    same values and launches): the whole quantized cache (all 8 x 16,384
    tokens' page entries, side rows and scales) byte for byte against the
    oracle's re-prefill, then the attention sampled at tokens around every
    region boundary of each chunk against the oracle's per-token attention."""
    from synth import draw_values
    wl = make_workload(4)
    nseq, n = wl.prefill_nseq, wl.prefill_len
    dev = torch.device("cuda")
    _say(f"[chunk] benchmark re-prefill {nseq} x {n}")
    pk, pv, _ = draw_values(wl.seed, 1000, nseq * n, 1, 4, wl.Hkv, device=dev)
    pq = draw_values(wl.seed, 1001, 1, nseq * n, wl.Hq, wl.Hkv, device=dev)[2]
    ppages = nseq * n // 16
    cache = kv4.Kv4Cache.zeros(ppages, wl.Hkv, nseq, dev)
    table = torch.arange(ppages, dtype=torch.int32, device=dev).view(nseq, n // 16)
    cu = torch.arange(0, nseq * n + 1, n, dtype=torch.int32, device=dev)
    start = torch.zeros(nseq, dtype=torch.int32, device=dev)
    slot = torch.arange(nseq, dtype=torch.int32, device=dev)
    kv4.prefill_quantize(cache, pk, pv, cu, start, slot, table, n)
    out, lse = kv4.prefill_attention(cache, pq, cu, start, slot, table, n, SCALE)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    hk = pk.view(torch.int16).cpu().numpy().view(np.uint16)
    hv = pv.view(torch.int16).cpu().numpy().view(np.uint16)
    hq = pq.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.Cache(ppages, wl.Hkv, nseq)
    oracle.prefill(ref, hk, hv, cu.cpu().numpy(), start.cpu().numpy(), slot.cpu().numpy(), table.cpu().numpy())
    assert np.array_equal(cache.pages.cpu().numpy(), ref.pages), "re-prefill page bytes differ"
    assert np.array_equal(cache.side_codes.cpu().numpy(), ref.side_codes), "re-prefill side codes differ"
    assert np.array_equal(cache.side_scales.cpu().numpy().view(np.uint16), ref.side_scales), \
        "re-prefill side scales differ"
    _say(f"[chunk] benchmark re-prefill: {ref.pages.nbytes >> 20} MiB of pages and all side rows equal")
    rng = np.random.default_rng(7)
    pos = [0, 15, 16, 31, 143, 144, 4095, n // 2 + 3, n - 129, n - 128, n - 127, n - 2, n - 1]
    tokens = np.array([s * n + p for s in (0, 3, 7) for p in pos], np.int64)
    heads = rng.integers(0, wl.Hq, len(tokens))
    r_out, r_lse = oracle.prefill_attention_sampled(ref, hq, cu.cpu().numpy(), start.cpu().numpy(),
                                                    slot.cpu().numpy(), table.cpu().numpy(), wl.Hq, SCALE,
                                                    tokens, heads)
    got_o = out.cpu().numpy()[tokens, heads]
    got_l = lse.cpu().numpy()[tokens, heads]
    err = float(np.abs(got_o - r_out).max())
    lerr = float(np.abs(got_l - r_lse).max())
    _say(f"[chunk] benchmark sample of {len(tokens)}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)
