"""Pins of the oracle's KV8-everywhere variant (the INT8 comparison of the
KV4-RL pages' quantization-target comparison, figure 3): every position is
stored as the side rows store protected positions (rotated keys, symmetric
INT8 per 128-dim vector, FP16 scale) and attended with the protected path's
arithmetic."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import make_workload
from tests.wl import host_inputs, oracle_cache

SCALE = 1.0 / math.sqrt(128)
LOG2E = 1.0 / math.log(2.0)


def kv8_cache(wl, hi):
    """Positions [0, ctx-1) by re-prefill, then this step's token appended."""
    cache = oracle.Kv8Cache(wl.num_pages, wl.Hkv)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    oracle.kv8_prefill(cache, k, v, cu, np.zeros(wl.B, np.int32), wl.page_table)
    ka, va = hi.at(wl.ctx - 1)
    oracle.kv8_append(cache, ka, va, (wl.ctx - 1).astype(np.int32), wl.page_table)
    return cache


@pytest.fixture(scope="module")
def small():
    wl = make_workload(0, ctx=[1, 16, 17, 40, 150, 205], Hq=4, Hkv=1, seed=41)
    hi = host_inputs(wl)
    return wl, hi, kv8_cache(wl, hi)


def _decode(wl, cache, hi, **kw):
    return oracle.kv8_decode(cache, hi.q, wl.ctx.astype(np.int32), wl.page_table, wl.Hq, SCALE, **kw)


def test_kv8_blocks_hold_int8_of_rotated_keys_and_values(small):
    wl, hi, cache = small
    for b in range(wl.B):
        for p in range(int(wl.ctx[b])):
            k = oracle.bf16_to_f32(hi.k[hi.offsets[b] + p])
            v = oracle.bf16_to_f32(hi.v[hi.offsets[b] + p])
            kr = (brute.fwht_f32_recursive(k) * brute.inv_sqrt128_f32()).astype(np.float32)
            k8, ks = oracle.quant_int8(kr)
            v8, vs = oracle.quant_int8(v)
            for g in range(wl.Hkv):
                kc, vc, sk, sv = brute.unpack_kv8_block(cache.pages[wl.page_table[b, p // 16], g])
                t = p % 16
                assert np.array_equal(kc[t], k8[g]) and np.array_equal(vc[t], v8[g])
                assert sk[t] == float(ks[g:g + 1].view(np.float16)[0])
                assert sv[t] == float(vs[g:g + 1].view(np.float16)[0])


def test_kv8_appends_equal_prefill(small):
    wl, hi, cache = small
    step = oracle.Kv8Cache(wl.num_pages, wl.Hkv)
    for p in range(int(wl.ctx.max())):
        live = np.nonzero(wl.ctx > p)[0]
        rows = hi.offsets[live] + p
        oracle.kv8_append(step, hi.k[rows], hi.v[rows], np.full(len(live), p, np.int32),
                          wl.page_table[live])
    assert np.array_equal(step.pages, cache.pages)


def test_kv8_decode_matches_brute_force(small):
    wl, hi, cache = small
    out, lse, dbg = _decode(wl, cache, hi, debug=True)
    sl = float(oracle.scale_log2(SCALE))
    for b in range(wl.B):
        for h in (0, 3):
            o, l, qk = brute.kv8_decode_one(cache.pages, hi.q[b, h], int(wl.ctx[b]), h // wl.group,
                                            wl.page_table[b], sl)
            assert np.abs(out[b, h] - o).max() < 1e-9
            assert abs(lse[b, h] - l) < 1e-9
            assert sorted(qk) == list(range(int(wl.ctx[b])))
            for p, d in qk.items():
                assert dbg["qk"][b, h, p] == d
            qc, _, qs = brute.query_codes(hi.q[b, h])
            assert np.array_equal(dbg["qcodes"][b, h], qc) and dbg["qsum"][b, h] == qs


def test_kv8_is_softmax_over_dequantized_rows(small):
    """FP64 softmax of the dequantized INT8 logits over every position, values
    v^ = bf16(s_v c) (exact in FP64): the FP32 weights differ by rounding only."""
    wl, hi, cache = small
    out, lse, _ = _decode(wl, cache, hi)
    for b in range(wl.B):
        for h in (1, 2):
            qc, s_q, _ = brute.query_codes(hi.q[b, h])
            z, vals = [], []
            for p in range(int(wl.ctx[b])):
                kc, vc, sk, sv = brute.unpack_kv8_block(cache.pages[wl.page_table[b, p // 16], 0])
                t = p % 16
                z.append(SCALE * LOG2E * s_q * sk[t] * float(qc @ kc[t]))
                vals.append([brute.rnbf16(sv[t] * float(c)) for c in vc[t]])
            z, vals = np.array(z), np.array(vals)
            e = np.exp2(z - z.max())
            assert np.abs(out[b, h] - (e[:, None] * vals).sum(0) / e.sum()).max() < 1e-4
            assert abs(lse[b, h] - math.log(2) * (z.max() + math.log2(e.sum()))) < 1e-4


def test_kv8_equals_kv4rl_when_every_position_is_protected():
    """With L <= s + w every KV4-RL position is in the protected region, whose
    INT8 rows hold the same codes as the KV8 pool: the two give the same bits."""
    wl = make_workload(0, ctx=[1, 15, 16, 17, 100, 144], Hq=8, Hkv=2, seed=42)
    hi = host_inputs(wl)
    o8, l8, _ = _decode(wl, kv8_cache(wl, hi), hi)
    o4, l4, _ = oracle.decode(oracle_cache(wl, hi), hi.q, wl.ctx.astype(np.int32), wl.slots,
                              wl.page_table, wl.Hq, SCALE)
    assert np.array_equal(o8, o4) and np.array_equal(l8, l4)


def test_kv8_page_permutation_invariance():
    wl_a = make_workload(0, ctx=[150, 333, 64], Hq=8, Hkv=2, seed=11)
    wl_b = make_workload(0, ctx=[150, 333, 64], Hq=8, Hkv=2, seed=11, pool_slack=9)
    hi = host_inputs(wl_a)
    oa, la, da = _decode(wl_a, kv8_cache(wl_a, hi), hi, debug=True)
    ob, lb, db = _decode(wl_b, kv8_cache(wl_b, hi), hi, debug=True)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    assert np.array_equal(da["qk"], db["qk"])
