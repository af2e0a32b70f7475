"""Pins of the oracle's protection budget beyond the default (s = 16 sink
positions, w = 128 recent positions): unprotected KV4 (s = w = 0), all-sink
(s = 144), all-recent (w = 144) and an intermediate split (s = 32, w = 64).

KV4-RL, sections on the protected region and on the budget allocation
(figures 3 and 4(b)): the same cache and decode step with the INT8 side
buffer holding the first s positions and a ring of the last w positions,
and the INT4 main region covering [s, L - w)."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import make_workload
from tests.wl import host_inputs, oracle_cache

SCALE = 1.0 / math.sqrt(128)
LOG2E = 1.0 / math.log(2.0)
BUDGETS = [(16, 128), (0, 0), (144, 0), (0, 144), (32, 64)]
CTX = [1, 17, 33, 100, 145, 170, 205, 300]


def _ids(b):
    return f"s{b[0]}w{b[1]}"


def _protected(L, s, w):
    return list(range(min(s, L))) + list(range(max(s, L - w), L))


def _row(p, s, w):
    return p if p < s else s + p % w


@pytest.fixture(scope="module", params=BUDGETS, ids=_ids)
def case(request):
    s, w = request.param
    wl = make_workload(0, ctx=CTX, Hq=4, Hkv=1, seed=21)
    hi = host_inputs(wl)
    return s, w, wl, hi, oracle_cache(wl, hi, sink=s, window=w)


def _decode(wl, cache, hi, **kw):
    return oracle.decode(cache, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq,
                         SCALE, **kw)


def test_budget_decode_matches_brute_force(case):
    s, w, wl, hi, cache = case
    out, lse, dbg = _decode(wl, cache, hi, debug=True)
    sl = float(oracle.scale_log2(SCALE))
    for b in range(wl.B):
        L = int(wl.ctx[b])
        for h in (0, 3):
            o, l, qk, pc, pv = brute.decode_one(cache.pages, cache.side_codes, cache.side_scales,
                                                wl.Hkv, hi.q[b, h], L, wl.slots[b], h // wl.group,
                                                wl.page_table[b], sl, sink=s, window=w)
            # every position is attended exactly once, main region = [s, L - w)
            assert sorted(qk) == list(range(L))
            assert sorted(pc) == list(range(s, max(s, L - w)))
            assert np.abs(out[b, h] - o).max() < 1e-9
            assert abs(lse[b, h] - l) < 1e-9
            for p, d in qk.items():
                assert dbg["qk"][b, h, p] == d, (b, h, p)
            for p, c in pc.items():
                assert dbg["pcode"][b, h, p] == c, (b, h, p)
            for j, acc in pv.items():
                assert np.array_equal(dbg["pv"][b, h, j], acc), (b, h, j)


def _dequant_union(wl, cache, hi, b, h, s, w):
    """FP64 logits and values of every attended position: side rows s*c for
    the protected positions, delta*c+m (keys in the rotated basis) for the
    main region, against the dequantized INT8 rotated query."""
    L = int(wl.ctx[b])
    g = h // wl.group
    qc, s_q, _ = brute.query_codes(hi.q[b, h])
    qhat = s_q * qc.astype(np.float64)
    prot = set(_protected(L, s, w))
    logits, values = [], []
    for p in range(L):
        if p in prot:
            r = _row(p, s, w)
            sc = cache.side_scales[wl.slots[b], g, r].view(np.float16).astype(np.float64)
            k = sc[0] * cache.side_codes[wl.slots[b], g, r, 0].astype(np.float64)
            v = np.array([brute.rnbf16(sc[1] * float(c)) for c in cache.side_codes[wl.slots[b], g, r, 1]])
        else:
            kc, vc, kd, km, vd, vm = brute.unpack_block(cache.pages[wl.page_table[b, p // 16], g])
            t = p % 16
            k = kd[t] * kc[t] + km[t]
            v = vd[t] * vc[t] + vm[t]
        logits.append(SCALE * LOG2E * float(qhat @ k))
        values.append(v)
    return np.array(logits), np.array(values)


def test_budget_exact_pv_is_single_softmax_over_union(case):
    s, w, wl, hi, cache = case
    out, lse, _ = _decode(wl, cache, hi, pv_exact=True)
    for b in range(wl.B):
        for h in (1, 2):
            z, v = _dequant_union(wl, cache, hi, b, h, s, w)
            e = np.exp2(z - z.max())
            assert np.abs(out[b, h] - (e[:, None] * v).sum(0) / e.sum()).max() < 1e-4
            assert abs(lse[b, h] - math.log(2) * (z.max() + math.log2(e.sum()))) < 1e-4


def test_budget_side_rows(case):
    """Sinks in rows [0, s), position p >= s in row s + (p mod w); rows no
    position reached stay untouched; w = 0 writes nothing past the sinks."""
    s, w, wl, hi, cache = case
    for b in range(wl.B):
        L = int(wl.ctx[b])
        written = set()
        for p in _protected(L, s, w):
            k = oracle.bf16_to_f32(hi.k[hi.offsets[b] + p])
            v = oracle.bf16_to_f32(hi.v[hi.offsets[b] + p])
            kr = (brute.fwht_f32_recursive(k) * brute.inv_sqrt128_f32()).astype(np.float32)
            k8, ks = oracle.quant_int8(kr)
            v8, vs = oracle.quant_int8(v)
            r = _row(p, s, w)
            written.add(r)
            sl = wl.slots[b]
            assert np.array_equal(cache.side_codes[sl, :, r, 0], k8)
            assert np.array_equal(cache.side_codes[sl, :, r, 1], v8)
            assert np.array_equal(cache.side_scales[sl, :, r, 0], ks)
            assert np.array_equal(cache.side_scales[sl, :, r, 1], vs)
        # a ring that wrapped holds exactly the recent window; others are untouched
        reached = set(range(min(s, L))) | {_row(p, s, w) for p in range(s, L)} if w else set(range(min(s, L)))
        assert written <= reached
        if L - s <= w or w == 0:
            assert reached == written
        for r in range(oracle.SIDE_ROWS):
            if r not in reached:
                assert not cache.side_codes[wl.slots[b], :, r].any(), (b, r)
                assert not cache.side_scales[wl.slots[b], :, r].any(), (b, r)


def test_budget_appends_equal_prefill(case):
    s, w, wl, hi, cache = case
    step = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, s, w)
    for p in range(int(wl.ctx.max())):
        live = np.nonzero(wl.ctx > p)[0]
        rows = hi.offsets[live] + p
        oracle.append(step, hi.k[rows], hi.v[rows], np.full(len(live), p, np.int32),
                      wl.slots[live], wl.page_table[live])
    assert np.array_equal(step.pages, cache.pages)
    assert np.array_equal(step.side_codes, cache.side_codes)
    assert np.array_equal(step.side_scales, cache.side_scales)


def test_budget_regions_read_disjointly(case):
    """Garbage in the INT4 entries of protected positions, and in every side
    row no protected position maps to, changes no output bit."""
    s, w, wl, hi, cache = case
    out0, lse0, _ = _decode(wl, cache, hi)
    rng = np.random.default_rng(3)
    c2 = cache.copy()
    for b in range(wl.B):
        L = int(wl.ctx[b])
        prot = _protected(L, s, w)
        live_rows = {_row(p, s, w) for p in prot}
        for r in range(oracle.SIDE_ROWS):
            if r not in live_rows:
                c2.side_codes[wl.slots[b], :, r] = rng.integers(-127, 128, c2.side_codes.shape[2:][1:],
                                                                dtype=np.int8)[None]
                c2.side_scales[wl.slots[b], :, r] = rng.integers(0, 0x7C00, 2, dtype=np.uint16)[None]
        for p in prot:
            blk = c2.pages[wl.page_table[b, p // 16], 0]
            t = p % 16
            blk[64 * t:64 * t + 64] = rng.integers(0, 256, 64)
            blk[2048 + 4 * t:2048 + 4 * t + 4] = rng.integers(0, 256, 4)
            blk[2112 + 4 * t:2112 + 4 * t + 4] = rng.integers(0, 256, 4)
            nib = rng.integers(0, 16, 128).astype(np.uint8)
            byte = blk[1024 + t // 2:2048:8]
            keep = 0xF0 if t % 2 == 0 else 0x0F
            blk[1024 + t // 2:2048:8] = (byte & keep) | (nib << (0 if t % 2 == 0 else 4))
    out1, lse1, _ = _decode(wl, c2, hi)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_full_budgets_agree_up_to_capacity():
    """With s + w = 144 and L <= 144 every position is protected and gathered
    in ascending order, so the three splits give the same bits."""
    wl = make_workload(0, ctx=[1, 16, 17, 100, 143, 144], Hq=4, Hkv=1, seed=4)
    hi = host_inputs(wl)
    res = [_decode(wl, oracle_cache(wl, hi, sink=s, window=w), hi) for s, w in
           ((16, 128), (144, 0), (0, 144), (64, 80))]
    for out, lse, _ in res[1:]:
        assert np.array_equal(out, res[0][0]) and np.array_equal(lse, res[0][1])


def test_unprotected_keeps_integer_path_for_every_position():
    """s = w = 0: every position goes through the INT4 tile path; the first
    tile starts at page 0 and the P-operand codes cover [0, L)."""
    wl = make_workload(0, ctx=[1, 16, 40], Hq=4, Hkv=1, seed=8)
    hi = host_inputs(wl)
    cache = oracle_cache(wl, hi, sink=0, window=0)
    assert not cache.side_codes.any() and not cache.side_scales.any()
    _, _, dbg = _decode(wl, cache, hi, debug=True)
    for b in range(wl.B):
        L = int(wl.ctx[b])
        for h in range(wl.Hq):
            # the largest weight of every tile quantizes to 127
            for j in range((L + 15) // 16):
                assert dbg["pcode"][b, h, 16 * j:min(L, 16 * j + 16)].max() == 127


@pytest.mark.parametrize("s,w", [(8, 0), (16, 129), (-16, 0), (0, -1), (160, 0)])
def test_invalid_budgets_rejected(s, w):
    with pytest.raises(ValueError):
        oracle.Cache(4, 1, 1, s, w)
    c = oracle.Cache(4, 1, 1)
    c.sink, c.window = s, w  # the C library checks as well
    with pytest.raises(ValueError):
        oracle.decode(c, np.zeros((1, 1, 128), np.uint16), np.array([1], np.int32), None,
                      np.zeros((1, 4), np.int32), 1, SCALE)
