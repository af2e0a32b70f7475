"""GPU parity at the full sizes of the benchmark workloads.

The whole batch is built and decoded on the GPU exactly as bench.py does it
(values drawn on the device, re-prefill of the leading positions, this
step's append, one decode launch over all B sequences in the timed launch
configuration).  The CPU oracle rebuilds the whole batch from the same values
in the same page table: every page block and side row bit-exact, out within
2e-3 and lse within 1e-4 for every sequence and head.  A sample of sequences
is also decoded by the oracle with its integer intermediates: query codes /
int32 QK / P-operand codes / int32 PV accumulators bit-exact.  The
benchmark's own launch, the one-launch step (this step's append inside the
decode), is checked the same way on the 256-sequence workload."""
import math

import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from synth import draw_values, make_workload
from tests.wl import bf16_bits

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4
SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _sample(ctx, n_random, seed):
    """Shortest, longest, median and a few random sequences."""
    order = np.argsort(ctx, kind="stable")
    rng = np.random.default_rng(seed)
    pick = {int(order[0]), int(order[-1]), int(order[len(order) // 2])}
    pick.update(int(i) for i in rng.choice(len(ctx), size=min(n_random, len(ctx)), replace=False))
    return np.array(sorted(pick))


def _build_gpu(wl, layer, dev, append=True):
    n_tok = int(wl.ctx.sum())
    k, v, q = draw_values(wl.seed, layer, n_tok, wl.B, wl.Hq, wl.Hkv, device=dev)
    off = np.zeros(wl.B + 1, np.int64)
    off[1:] = np.cumsum(wl.ctx)
    lead = wl.ctx - 1 if wl.append_step else wl.ctx
    rows = torch.from_numpy(np.concatenate([np.arange(off[b], off[b] + lead[b]) for b in range(wl.B)])).to(dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)).to(dev)
    table = torch.from_numpy(wl.page_table).to(dev)
    slots = torch.from_numpy(wl.slots).to(dev)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev)
    kv4.prefill_quantize(cache, k[rows].contiguous(), v[rows].contiguous(), cu,
                         torch.zeros(wl.B, dtype=torch.int32, device=dev), slots, table, int(lead.max()))
    if wl.append_step and append:
        last = torch.from_numpy(off[:-1] + lead).to(dev)
        kv4.append(cache, k[last].contiguous(), v[last].contiguous(),
                   torch.from_numpy((wl.ctx - 1).astype(np.int32)).to(dev), slots, table)
    return cache, k, v, q, off, table, slots


def _oracle_full(wl, k, v, q, off):
    """The oracle's cache of the whole batch in the workload's own page table
    and slots (re-prefill of the leading positions, then this step's token),
    and its decode of every sequence and head (out, lse)."""
    lead = wl.ctx - 1 if wl.append_step else wl.ctx
    kh, vh = bf16_bits(k), bf16_bits(v)
    rows = np.concatenate([np.arange(off[b], off[b] + lead[b]) for b in range(wl.B)])
    cu = np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots)
    oracle.prefill(cache, kh[rows], vh[rows], cu, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    del rows
    if wl.append_step:
        last = off[:-1] + lead
        oracle.append(cache, kh[last], vh[last], lead.astype(np.int32), wl.slots, wl.page_table)
    del kh, vh
    out, lse, _ = oracle.decode(cache, bf16_bits(q), wl.ctx.astype(np.int32), wl.slots, wl.page_table,
                                wl.Hq, SCALE)
    return cache, out, lse


def _compare_full(cache, out, lse, ref, ref_out, ref_lse, what):
    assert np.array_equal(cache.pages.cpu().numpy(), ref.pages), f"{what}: page bytes differ"
    assert np.array_equal(cache.side_codes.cpu().numpy(), ref.side_codes), f"{what}: side codes differ"
    assert np.array_equal(cache.side_scales.cpu().numpy().view(np.uint16), ref.side_scales), \
        f"{what}: side scales differ"
    err = float(np.abs(out.cpu().numpy() - ref_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    _say(f"{what}: every sequence and head: out {err:.2e} lse {lerr:.2e}; pages and side rows equal")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (what, err, lerr)


def _oracle_for(wl, sample, k, v, q, off):
    """Oracle cache and decode of the sampled sequences, from the device values."""
    ctx = wl.ctx[sample]
    need = (ctx + 15) // 16
    table = np.zeros((len(sample), int(need.max())), np.int32)
    o = 0
    for i, n in enumerate(need):
        table[i, :n] = np.arange(o, o + n)
        o += n
    lead = ctx - 1 if wl.append_step else ctx
    rows_all = np.concatenate([np.arange(off[b], off[b] + wl.ctx[b]) for b in sample])
    kh = bf16_bits(k[torch.from_numpy(rows_all).to(k.device)])
    vh = bf16_bits(v[torch.from_numpy(rows_all).to(v.device)])
    soff = np.zeros(len(sample) + 1, np.int64)
    soff[1:] = np.cumsum(ctx)
    lrows = np.concatenate([np.arange(soff[i], soff[i] + lead[i]) for i in range(len(sample))])
    cu = np.concatenate([[0], np.cumsum(lead)]).astype(np.int32)
    slots = np.arange(len(sample), dtype=np.int32)
    cache = oracle.Cache(int(need.sum()), wl.Hkv, len(sample))
    oracle.prefill(cache, kh[lrows], vh[lrows], cu, np.zeros(len(sample), np.int32), slots, table)
    if wl.append_step:
        last = soff[:-1] + lead
        oracle.append(cache, kh[last], vh[last], lead.astype(np.int32), slots, table)
    qh = bf16_bits(q[torch.from_numpy(sample).to(q.device)])
    out, lse, dbg = oracle.decode(cache, qh, ctx.astype(np.int32), slots, table, wl.Hq, SCALE, debug=True)
    return cache, table, out, lse, dbg


@pytest.mark.parametrize("index,layer", [(2, 0), (3, 0), (4, 0), (4, 35)])
def test_fullsize_sampled_parity(index, layer):
    dev = torch.device("cuda")
    wl = make_workload(index)
    _say(f"[fullsize] workload {wl.name} B={wl.B} layer {layer} mean ctx {wl.ctx.mean():.0f} max {wl.ctx.max()}")
    cache, k, v, q, off, table, slots = _build_gpu(wl, layer, dev)
    ctx_d = torch.from_numpy(wl.ctx.astype(np.int32)).to(dev)
    max_ctx = int(wl.ctx.max())
    out, lse = kv4.decode_attention(cache, q, ctx_d, slots, table, max_ctx, SCALE)
    out_d, lse_d, dbg = kv4.decode_attention_debug(cache, q, ctx_d, slots, table, max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    _say("[fullsize] oracle on the whole batch")
    ref_all, out_all, lse_all = _oracle_full(wl, k, v, q, off)
    _compare_full(cache, out, lse, ref_all, out_all, lse_all, f"[fullsize] {wl.name} layer {layer}")
    del ref_all, out_all, lse_all
    sample = _sample(wl.ctx, 5, 100 + index + layer)
    _say(f"[fullsize] oracle on sequences {sample.tolist()} (ctx {wl.ctx[sample].tolist()})")
    ref, rtable, ref_out, ref_lse, ref_dbg = _oracle_for(wl, sample, k, v, q, off)

    pages = cache.pages
    for i, b in enumerate(sample):
        n = int((wl.ctx[b] + 15) // 16)
        got = pages[torch.from_numpy(wl.page_table[b, :n].astype(np.int64)).to(dev)].cpu().numpy()
        want = ref.pages[rtable[i, :n]]
        assert np.array_equal(got, want), f"pages of sequence {b} differ"
        assert np.array_equal(cache.side_codes[int(wl.slots[b])].cpu().numpy(), ref.side_codes[i])
        assert np.array_equal(cache.side_scales[int(wl.slots[b])].cpu().numpy().view(np.uint16),
                              ref.side_scales[i])
    sel = torch.from_numpy(sample).to(dev)
    for key in ("qcodes", "qsum"):
        assert np.array_equal(dbg[key][sel].cpu().numpy(), ref_dbg[key]), key
    for i, b in enumerate(sample):
        L = int(wl.ctx[b])
        n = (L + 15) // 16
        for key in ("qk", "pcode"):
            got = dbg[key][int(b), :, :L].cpu().numpy()
            assert np.array_equal(got, ref_dbg[key][i, :, :L]), f"{key} of sequence {b}"
        got = dbg["pv"][int(b), :, :n].cpu().numpy()
        assert np.array_equal(got, ref_dbg["pv"][i, :, :n]), f"pv of sequence {b}"
    err = float(np.abs(out[sel].cpu().numpy() - ref_out).max())
    lerr = float(np.abs(lse[sel].cpu().numpy() - ref_lse).max())
    _say(f"[fullsize] {wl.name} layer {layer}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (err, lerr)
    # every output is finite and every lse at least the largest logit seen by any region
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("layer", [0, 35])
def test_fullsize_one_launch_step(layer):
    """The launch bench.py times: kv4_append_decode_attention on the
    256-sequence workload (re-prefill of [0, ctx-1), then this step's append
    inside the decode), against the oracle's append + decode of the whole
    batch: every page block and side row bit-exact, every out and lse within
    the bar."""
    dev = torch.device("cuda")
    wl = make_workload(4)
    _say(f"[fullsize] one-launch step, workload {wl.name} layer {layer}")
    cache, k, v, q, off, table, slots = _build_gpu(wl, layer, dev, append=False)
    last = torch.from_numpy(off[:-1] + wl.ctx - 1).to(dev)
    ctx_d = torch.from_numpy(wl.ctx.astype(np.int32)).to(dev)
    out, lse = kv4.append_decode_attention(cache, k[last].contiguous(), v[last].contiguous(), ctx_d - 1, q,
                                           ctx_d, slots, table, int(wl.ctx.max()), SCALE)
    torch.cuda.synchronize()
    ref, ref_out, ref_lse = _oracle_full(wl, k, v, q, off)
    _compare_full(cache, out, lse, ref, ref_out, ref_lse, f"[fullsize] one-launch step layer {layer}")


@pytest.mark.parametrize("first", [0, 9, 18, 27])
def test_benchmark_workload_every_layer(first):
    """All 36 layers of the 256-sequence benchmark workload, built and decoded
    on the GPU as bench.py does (each layer its own values and cache); per
    layer the shortest sequence and one drawn at random are rebuilt by the
    oracle: their pages, side rows and query codes bit-exact, out and lse
    within the bar."""
    dev = torch.device("cuda")
    wl = make_workload(4)
    order = np.argsort(wl.ctx, kind="stable")
    for layer in range(first, first + 9):
        cache, k, v, q, off, table, slots = _build_gpu(wl, layer, dev)
        ctx_d = torch.from_numpy(wl.ctx.astype(np.int32)).to(dev)
        out, lse = kv4.decode_attention(cache, q, ctx_d, slots, table, int(wl.ctx.max()), SCALE)
        torch.cuda.synchronize()
        rng = np.random.default_rng(1000 + layer)
        sample = np.unique([int(order[0]), int(rng.integers(wl.B))])
        ref, rtable, ref_out, ref_lse, ref_dbg = _oracle_for(wl, sample, k, v, q, off)
        for i, b in enumerate(sample):
            n = int((wl.ctx[b] + 15) // 16)
            got = cache.pages[torch.from_numpy(wl.page_table[b, :n].astype(np.int64)).to(dev)].cpu().numpy()
            assert np.array_equal(got, ref.pages[rtable[i, :n]]), f"layer {layer}: pages of {b}"
            assert np.array_equal(cache.side_codes[int(wl.slots[b])].cpu().numpy(), ref.side_codes[i])
        sel = torch.from_numpy(sample).to(dev)
        err = float(np.abs(out[sel].cpu().numpy() - ref_out).max())
        lerr = float(np.abs(lse[sel].cpu().numpy() - ref_lse).max())
        _say(f"[layers] layer {layer} sequences {sample.tolist()}: out {err:.2e} lse {lerr:.2e}")
        assert err <= OUT_TOL and lerr <= LSE_TOL, (layer, err, lerr)
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        del cache, k, v, q
