"""Pins of the oracle's decode step against brute force, closed forms and
invariants (no GPU)."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import make_workload
from tests import crafted
from tests.wl import host_inputs, oracle_cache

SCALE = 1.0 / math.sqrt(128)
LOG2E = 1.0 / math.log(2.0)


def _decode(wl, cache, hi, **kw):
    return oracle.decode(cache, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq,
                         SCALE, **kw)


def _dequant_union(wl, cache, hi, b, h):
    """FP64 logits and values of every attended position from dequantized
    codes: main region delta*c+m (K in the rotated basis), protected region
    s*c; the query is the dequantized INT8 rotated query."""
    L = int(wl.ctx[b])
    g = h // wl.group
    qc, s_q, _ = brute.query_codes(hi.q[b, h])
    qhat = s_q * qc.astype(np.float64)
    logits, values = [], []
    for p in range(L):
        if p < 16 or p >= max(16, L - 128):
            row = p if p < 16 else 16 + p % 128
            s = cache.side_scales[wl.slots[b], g, row].view(np.float16).astype(np.float64)
            k = s[0] * cache.side_codes[wl.slots[b], g, row, 0].astype(np.float64)
            v = np.array([brute.rnbf16(s[1] * float(c)) for c in cache.side_codes[wl.slots[b], g, row, 1]])
        else:
            kc, vc, kd, km, vd, vm = brute.unpack_block(cache.pages[wl.page_table[b, p // 16], g])
            t = p % 16
            k = kd[t] * kc[t] + km[t]
            v = vd[t] * vc[t] + vm[t]
        logits.append(SCALE * LOG2E * float(qhat @ k))
        values.append(v)
    return np.array(logits), np.array(values)


@pytest.fixture(scope="module")
def small():
    wl = make_workload(0, ctx=[1, 17, 145, 170, 205], Hq=4, Hkv=1)
    hi = host_inputs(wl)
    cache = oracle_cache(wl, hi)
    return wl, hi, cache


def test_decode_matches_brute_force(small):
    wl, hi, cache = small
    out, lse, dbg = _decode(wl, cache, hi, debug=True)
    sl = oracle.scale_log2(SCALE)
    for b in range(wl.B):
        for h in (0, 3):
            o, l, qk, pc, pv = brute.decode_one(cache.pages, cache.side_codes, cache.side_scales,
                                                wl.Hkv, hi.q[b, h], int(wl.ctx[b]), wl.slots[b],
                                                h // wl.group, wl.page_table[b], float(sl))
            assert np.abs(out[b, h] - o).max() < 1e-9
            assert abs(lse[b, h] - l) < 1e-9
            for p, d in qk.items():
                assert dbg["qk"][b, h, p] == d, (b, h, p)
            for p, c in pc.items():
                assert dbg["pcode"][b, h, p] == c, (b, h, p)
            for j, acc in pv.items():
                assert np.array_equal(dbg["pv"][b, h, j], acc), (b, h, j)
            qc, _, qs = brute.query_codes(hi.q[b, h])
            assert np.array_equal(dbg["qcodes"][b, h], qc) and dbg["qsum"][b, h] == qs


def test_merge_equals_single_softmax_over_union(small):
    wl, hi, cache = small
    out_x, lse_x, _ = _decode(wl, cache, hi, pv_exact=True)
    out_r, lse_r, _ = _decode(wl, cache, hi)
    for b in range(wl.B):
        for h in range(wl.Hq):
            z, v = _dequant_union(wl, cache, hi, b, h)
            w = np.exp2(z - z.max())
            want = (w[:, None] * v).sum(0) / w.sum()
            want_lse = math.log(2) * (z.max() + math.log2(w.sum()))
            # FP32 logits vs FP64 logits: relative 1e-6 in the weights
            assert np.abs(out_x[b, h] - want).max() < 1e-4
            assert abs(lse_x[b, h] - want_lse) < 1e-4
            # the normaliser uses unquantized weights: lse does not depend on the PV rule
            assert lse_r[b, h] == lse_x[b, h]


def test_pv_rule_error_bound(small):
    wl, hi, cache = small
    out_x, _, _ = _decode(wl, cache, hi, pv_exact=True)
    out_r, _, _ = _decode(wl, cache, hi)
    for b in range(wl.B):
        L = int(wl.ctx[b])
        g = 0
        # |s_u*uc - u| <= s_u/2 with s_u <= max delta_v / 127, and the tile weights
        # sum to at most the normaliser: the per-channel error is bounded by
        # max over tiles of (max delta_v) * sum_t cv / 254.
        bound = 0.0
        for j in range(1, (L - 128 - 1) // 16 + 1 if L > 144 else 1):
            kc, vc, kd, km, vd, vm = brute.unpack_block(cache.pages[wl.page_table[b, j], g])
            n = min(16, L - 128 - 16 * j)
            bound = max(bound, max(vd[:n]) * vc[:n].sum(0).max() / 254.0)
        err = np.abs(out_r[b] - out_x[b]).max()
        assert err <= bound * (1 + 1e-6) + 1e-12
        if L <= 144:
            assert err == 0.0


def test_single_position_context():
    wl = make_workload(0, ctx=[1, 1], Hq=4, Hkv=1)
    hi = host_inputs(wl)
    cache = oracle_cache(wl, hi)
    out, lse, _ = _decode(wl, cache, hi)
    for b in range(2):
        s = cache.side_scales[b, 0, 0].view(np.float16).astype(np.float64)
        vhat = np.array([brute.rnbf16(float(np.float32(s[1]) * np.float32(c)))
                         for c in cache.side_codes[b, 0, 0, 1]])
        z, _ = _dequant_union(wl, cache, hi, b, 0)
        for h in range(4):
            assert np.array_equal(out[b, h], vhat)
            zz, _ = _dequant_union(wl, cache, hi, b, h)
            assert abs(lse[b, h] - math.log(2) * zz[0]) < 1e-5 * max(1.0, abs(zz[0]))


def test_protected_region_is_textbook_softmax_on_grid_exact_codes():
    rng = np.random.default_rng(5)
    wl = make_workload(0, ctx=[40, 144], Hq=4, Hkv=1)
    hi = host_inputs(wl)
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots)
    cache.side_codes[:] = rng.integers(-127, 128, cache.side_codes.shape, dtype=np.int8)
    pow2 = np.float16(2.0) ** rng.integers(-8, -3, cache.side_scales.shape).astype(np.float16)
    cache.side_scales[:] = pow2.view(np.uint16)
    cache.pages[:] = rng.integers(0, 256, cache.pages.shape, dtype=np.uint8)  # must be ignored
    out, lse, _ = _decode(wl, cache, hi)
    for b in range(wl.B):
        for h in range(wl.Hq):
            L = int(wl.ctx[b])
            qc, s_q, _ = brute.query_codes(hi.q[b, h])
            rows = [p if p < 16 else 16 + p % 128 for p in range(L)]
            sk = cache.side_scales[b, 0, rows, 0].view(np.float16).astype(np.float64)
            sv = cache.side_scales[b, 0, rows, 1].view(np.float16).astype(np.float64)
            K = sk[:, None] * cache.side_codes[b, 0, rows, 0].astype(np.float64)
            V = sv[:, None] * cache.side_codes[b, 0, rows, 1].astype(np.float64)  # exact in BF16
            logits = SCALE * (K @ (s_q * qc.astype(np.float64)))
            w = np.exp(logits - logits.max())
            assert np.abs(out[b, h] - (w[:, None] * V).sum(0) / w.sum()).max() < 2e-5
            assert abs(lse[b, h] - (logits.max() + math.log(w.sum()))) < 1e-5


def test_regions_are_read_disjointly(small):
    """The two regions are read disjointly: garbage written into the INT4
    entries (codes, nibbles and metadata) of every sink and recent position
    changes no output bit.  (At L <= 144 that is every INT4 entry.)"""
    wl, hi, cache = small
    out0, lse0, _ = _decode(wl, cache, hi)
    rng = np.random.default_rng(9)
    c2 = cache.copy()
    for b in range(wl.B):
        L = int(wl.ctx[b])
        for p in list(range(min(16, L))) + list(range(max(16, L - 128), L)):
            blk = c2.pages[wl.page_table[b, p // 16], 0]
            t = p % 16
            blk[64 * t:64 * t + 64] = rng.integers(0, 256, 64)
            blk[2048 + 4 * t:2048 + 4 * t + 4] = rng.integers(0, 256, 4)
            blk[2112 + 4 * t:2112 + 4 * t + 4] = rng.integers(0, 256, 4)
            nib = rng.integers(0, 16, 128).astype(np.uint8)
            byte = blk[1024 + t // 2:2048:8]
            keep = 0xF0 if t % 2 == 0 else 0x0F
            blk[1024 + t // 2:2048:8] = (byte & keep) | (nib << (0 if t % 2 == 0 else 4))
        # pages wholly inside the protected region, and every page when L <= 144
    out1, lse1, _ = _decode(wl, c2, hi)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_page_permutation_invariance():
    wl_a = make_workload(0, ctx=[150, 333, 64], Hq=8, Hkv=2, seed=11)
    wl_b = make_workload(0, ctx=[150, 333, 64], Hq=8, Hkv=2, seed=11, pool_slack=9)
    assert not np.array_equal(wl_a.page_table, wl_b.page_table)
    hi = host_inputs(wl_a)
    ca, cb = oracle_cache(wl_a, hi), oracle_cache(wl_b, hi)
    oa, la, da = _decode(wl_a, ca, hi, debug=True)
    ob, lb, db = _decode(wl_b, cb, hi, debug=True)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    for key in da:
        assert np.array_equal(da[key], db[key]), key


def test_integer_accumulators_equal_fp64_sums(small):
    wl, hi, cache = small
    _, _, dbg = _decode(wl, cache, hi, debug=True)
    for b in range(wl.B):
        L = int(wl.ctx[b])
        for p in range(16, L - 128):
            kc, *_ = brute.unpack_block(cache.pages[wl.page_table[b, p // 16], 0])
            for h in range(wl.Hq):
                want = float(dbg["qcodes"][b, h].astype(np.float64) @ kc[p % 16].astype(np.float64))
                assert dbg["qk"][b, h, p] == want
                assert abs(want) <= 128 * 127 * 15



def _crafted_run(name):
    cache = oracle.Cache(2, 1, 1, sink=0, window=0)
    cache.pages[0, 0] = crafted.page(name)
    q = crafted.unit_query(1, 4)
    table = np.array([[0, 1]], np.int32)
    dec = oracle.decode(cache, q, np.array([16], np.int32), np.array([0], np.int32), table, 4, SCALE, debug=True)
    # the one-token chunk at the last position sees the same tile
    pre = oracle.prefill_attention(cache, q, np.array([0, 1], np.int32), np.array([15], np.int32),
                                   np.array([0], np.int32), table, 4, SCALE, debug=True)
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        assert np.array_equal(dec[2][key], pre[2][key]), key
    assert np.array_equal(dec[0], pre[0]) or np.abs(dec[0] - pre[0]).max() < 1e-12
    return dec


def _logit_units():
    """Base-2 logit of one unit of m_k for the unit query: S_q * c_q, with
    c_q = s_q * scale_log2 in FP32 (s_q = 2^-3.5 / 127)."""
    s_q = np.float32(np.float32(2.0 ** -3.5) / np.float32(127.0))
    return np.float32(s_q * np.float32(SCALE * LOG2E)), 127 * 128


def test_p_codes_when_127_over_u_max_overflows():
    """P-operand rule at its overflow corner: u_max FP32-subnormal, so
    127 / u_max is infinite; the nonzero u saturate at 127 and the zero
    weight's 0 * inf is read as code 0.  Position 0 carries all but 2^-111 of
    the weight, so out is its dequantized value m_v and lse its logit times
    ln 2."""
    mk0, _, _, _, mv0, _, code = crafted.CASES["u_max_subnormal"]
    out, lse, dbg = _crafted_run("u_max_subnormal")
    assert (dbg["qsum"] == 127 * 128).all()
    assert (dbg["pcode"][0, :, 0] == 0).all() and (dbg["pcode"][0, :, 1:16] == 127).all()
    assert (dbg["pv"][0, :, 0] == 15 * 127 * code).all()
    assert np.abs(out - mv0).max() < 1e-9
    c_q, S = _logit_units()
    z0 = np.float32(np.float32(mk0 * S) * c_q)
    assert np.abs(lse - math.log(2.0) * float(z0)).max() < 1e-5


def test_p_codes_when_weights_fall_below_the_exp2s_cutoff():
    """Positions 144 base-2 units below the maximum get e = 0 exactly (exp2s
    returns 0 below -125): codes 127 at position 0 and 0 elsewhere, and out
    is position 0's dequantized value delta_v * code + m_v."""
    mk0, _, dv0, _, mv0, _, code = crafted.CASES["weights_cut_off"]
    out, lse, dbg = _crafted_run("weights_cut_off")
    assert (dbg["pcode"][0, :, 0] == 127).all() and (dbg["pcode"][0, :, 1:16] == 0).all()
    assert (dbg["pv"][0, :, 0] == 127 * code).all()
    assert np.abs(out - (dv0 * code + mv0)).max() < 1e-9
    c_q, S = _logit_units()
    assert np.abs(lse - math.log(2.0) * float(np.float32(np.float32(mk0 * S) * c_q))).max() < 1e-5


def test_p_codes_when_every_v_vector_is_constant():
    """delta_v = 0 at every position: u_max = 0, every code 0, PV = 0, and
    out is the softmax-weighted mean of the offsets m_v (weights 2^(z - z_max)
    from the hand-computed logits)."""
    mk0, mk1, _, _, mv0, mv1, _ = crafted.CASES["u_max_zero"]
    out, lse, dbg = _crafted_run("u_max_zero")
    assert (dbg["pcode"][0, :, :16] == 0).all() and (dbg["pv"][0, :, 0] == 0).all()
    c_q, S = _logit_units()
    z0, z1 = (float(np.float32(np.float32(m * S) * c_q)) for m in (mk0, mk1))
    w = 2.0 ** (z1 - z0)
    want = (mv0 + 15 * w * mv1) / (1 + 15 * w)
    assert np.abs(out - want).max() < 1e-6
    assert np.abs(lse - math.log(2.0) * (z0 + math.log2(1 + 15 * w))).max() < 1e-5
