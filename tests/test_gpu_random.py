"""Seeded random cases on the GPU against the oracle: random batch sizes, head
counts, context lengths (many on a region boundary), protection budgets, slot
permutations and page pools with free pages, for the decode step (plain, and
with this step's append in the same launch), for re-prefill attention, and
for the MXFP4 and KV8 formats.  Bar: page blocks and side rows, query codes and sums, int32 QK, P codes and
int32 PV bit-exact; out within 2e-3 max-abs, lse within 1e-4."""
import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from synth import make_workload
from tests.gpu_util import SCALE, GpuCase, bf, i32
from tests.test_gpu_parity import assert_cache_equal
from tests.wl import host_inputs, oracle_cache

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4
BUDGETS = [(16, 128), (0, 0), (144, 0), (0, 144), (32, 64), (48, 96), (16, 0), (0, 16)]
# windows that are not a multiple of the page size: the boundary between the
# INT4 and the INT8 regions falls inside a page (seeds from 100 on); with
# w < 16 this step's token can share a page with the last main positions
ODD_BUDGETS = [(16, 100), (0, 7), (32, 1), (0, 15), (16, 113), (48, 17)]
EDGES = [1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 143, 144, 145, 160, 161, 176, 177]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _random_workload(seed):
    """A tiny-config workload with random shape, slots and a pool with free pages."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 20))
    Hkv = int(rng.choice([1, 2, 4]))
    ctx = np.where(rng.random(B) < 0.5, rng.choice(EDGES, B), rng.integers(1, 1200, B))
    wl = make_workload(0, seed=7000 + seed, ctx=ctx, Hq=4 * Hkv, Hkv=Hkv, pool_slack=int(rng.integers(1, 24)))
    extra = int(rng.integers(0, 5))
    wl.slots = rng.permutation(B + extra)[:B].astype(np.int32)
    wl.max_slots = B + extra
    pool = ODD_BUDGETS if seed >= 100 else BUDGETS
    sink, window = pool[int(rng.integers(0, len(pool)))] if seed < 100 else pool[seed % len(pool)]
    return wl, sink, window


def _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg):
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        got = dbg[key].cpu().numpy()
        bad = np.argwhere(got != r_dbg[key])
        assert len(bad) == 0, f"{tag} {key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[random] {tag}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


@pytest.mark.parametrize("seed", list(range(8)) + list(range(22, 34)) + list(range(100, 106)))
def test_random_decode(seed):
    wl, sink, window = _random_workload(seed)
    tag = f"decode seed {seed} B={wl.B} Hkv={wl.Hkv} s={sink} w={window} ctx max {int(wl.ctx.max())}"
    _say(f"[random] {tag}")
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi, sink=sink, window=window)
    case = GpuCase(wl, hi, sink=sink, window=window)
    out, lse, dbg = case.decode(debug=True)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    r_out, r_lse, r_dbg = oracle.decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq,
                                        SCALE, debug=True)
    _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg)


@pytest.mark.parametrize("seed", list(range(8, 14)) + list(range(34, 42)) + list(range(106, 118)))
def test_random_fused_step(seed):
    """This step's append inside the decode launch, from a cache holding
    [0, ctx - 1): pages, side rows, out and lse against the oracle's append
    followed by its decode."""
    wl, sink, window = _random_workload(seed)
    tag = f"fused seed {seed} B={wl.B} Hkv={wl.Hkv} s={sink} w={window}"
    _say(f"[random] {tag}")
    dev = torch.device("cuda")
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi, sink=sink, window=window)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, sink, window)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    if len(k):
        kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev), slots, table,
                             int(max(1, lead.max())))
    ka, va = hi.at(lead)
    out, lse = kv4.append_decode_attention(cache, bf(ka, dev), bf(va, dev), i32(lead, dev), bf(hi.q, dev),
                                           i32(wl.ctx, dev), slots, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pages.cpu().numpy(), ref.pages), tag
    assert np.array_equal(cache.side_codes.cpu().numpy(), ref.side_codes), tag
    assert np.array_equal(cache.side_scales.cpu().numpy().view(np.uint16), ref.side_scales.view(np.uint16)), tag
    r_out, r_lse, _ = oracle.decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[random] {tag}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


@pytest.mark.parametrize("seed", list(range(14, 22)) + list(range(42, 50)) + list(range(118, 124)) +
                         list(range(200, 220)))
def test_random_prefill_attention(seed):
    """Chunks of random length at the end of random prefixes (several per
    call), random budget and slots."""
    rng = np.random.default_rng(6000 + seed)
    wl, sink, window = _random_workload(seed)
    n = np.minimum(wl.ctx, rng.integers(1, 90, wl.B)).astype(np.int32)
    tag = f"re-prefill seed {seed} nseq={wl.B} Hkv={wl.Hkv} s={sink} w={window} tokens {int(n.sum())}"
    _say(f"[random] {tag}")
    dev = torch.device("cuda")
    hi = host_inputs(wl)
    k, v, cu_all = hi.prefix(wl.ctx)
    ref = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    oracle.prefill(ref, k, v, cu_all, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, sink, window)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu_all, dev), i32(np.zeros(wl.B), dev), slots, table,
                         int(wl.ctx.max()))
    start = (wl.ctx - n).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(cu[-1])
    qr = np.random.default_rng(seed).standard_normal((T, wl.Hq, 128)).astype(np.float32)
    q = torch.from_numpy(qr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out, lse, dbg = kv4.prefill_attention_debug(cache, bf(q, dev), i32(cu, dev), i32(start, dev), slots, table,
                                                int(wl.ctx.max()), SCALE)
    torch.cuda.synchronize()
    r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE,
                                                   debug=True)
    _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg)


@pytest.mark.parametrize("seed", range(50, 58))
def test_random_mx(seed):
    """MXFP4 main region with the random budget: page blocks and side rows
    bit-exact, out and lse within the bar."""
    from tests.test_gpu_mx import _Case, _oracle_mx
    wl, sink, window = _random_workload(seed)
    tag = f"mxfp4 seed {seed} B={wl.B} Hkv={wl.Hkv} s={sink} w={window}"
    _say(f"[random] {tag}")
    dev = torch.device("cuda")
    hi = host_inputs(wl)
    ref = _oracle_mx(wl, hi, sink, window)
    case = _Case(wl, hi, sink, window, dev)
    out, lse = kv4.mx_decode_attention(case.cache, bf(hi.q, dev), i32(wl.ctx, dev), case.slots, case.table,
                                       wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    r_out, r_lse = oracle.mx_decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[random] {tag}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


@pytest.mark.parametrize("seed", range(58, 66))
def test_random_kv8(seed):
    """KV8 everywhere on the random shapes (no budget): pool bytes, query
    codes and QK bit-exact, out and lse within the bar."""
    from tests.test_gpu_kv8 import _check
    wl, _, _ = _random_workload(seed)
    tag = f"kv8 seed {seed} B={wl.B} Hkv={wl.Hkv} ctx max {int(wl.ctx.max())}"
    _say(f"[random] {tag}")
    err, lerr = _check(wl, host_inputs(wl), torch.device("cuda"))
    _say(f"[random] {tag}: out {err:.2e} lse {lerr:.2e}")


def test_large_batch_short_contexts():
    """Many sequences (3000, above the 256 the in-kernel plan covers, so the
    plan kernel runs) with contexts drawn half from the region edges and half
    from [1, 400]: the decode and the one-launch step against the oracle."""
    rng = np.random.default_rng(4242)
    B = 3000
    ctx = np.where(rng.random(B) < 0.5, rng.choice(EDGES, B), rng.integers(1, 400, B))
    wl = make_workload(0, seed=4243, ctx=ctx, Hq=4, Hkv=1, pool_slack=8)
    tag = f"large batch B={wl.B} ctx max {int(wl.ctx.max())}"
    _say(f"[random] {tag}")
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi)
    case = GpuCase(wl, hi)
    out, lse, dbg = case.decode(debug=True)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    r_out, r_lse, r_dbg = oracle.decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq,
                                        SCALE, debug=True)
    _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg)
    # the one-launch step from a cache holding [0, ctx - 1)
    dev = torch.device("cuda")
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    if len(k):
        kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev), slots, table,
                             int(max(1, lead.max())))
    ka, va = hi.at(lead)
    out2, lse2 = kv4.append_decode_attention(cache, bf(ka, dev), bf(va, dev), i32(lead, dev), bf(hi.q, dev),
                                             i32(wl.ctx, dev), slots, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pages.cpu().numpy(), ref.pages)
    err = float(np.abs(out2.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse2.cpu().numpy() - r_lse).max())
    _say(f"[random] {tag} one launch: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL
