"""Pins of the oracle's MXFP4 variant (KV4-RL pages, comparison of 4-bit
formats, appendix D.4): the main region stored in OCP MXFP4 (32-element
blocks of E2M1 codes with an E8M0 scale, 4.25 bits per element), the rest of
KV4-RL unchanged."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import make_workload
from tests.wl import host_inputs, oracle_cache

SCALE = 1.0 / math.sqrt(128)
LOG2E = 1.0 / math.log(2.0)


def mx_cache(wl, hi, sink=16, window=128):
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    oracle.mx_prefill(cache, k, v, cu, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    ka, va = hi.at(wl.ctx - 1)
    oracle.mx_append(cache, ka, va, (wl.ctx - 1).astype(np.int32), wl.slots, wl.page_table)
    return cache


def _bf16(x):
    import torch
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _one_token(vrow):
    """Cache of one position whose value vector (kv-head 0) is vrow; K zero.
    Unprotected (s = w = 0): the INT8 side copy's FP16 scale could not hold
    the extreme values used here."""
    cache = oracle.Cache(1, 1, 1, 0, 0)
    v = _bf16(vrow).reshape(1, 1, 128)
    k = _bf16(np.zeros(128)).reshape(1, 1, 128)
    oracle.mx_append(cache, k, v, np.array([0], np.int32), np.array([0], np.int32), np.zeros((1, 1), np.int32))
    blk = cache.pages[0, 0]
    codes = [(int(blk[1024 + 8 * j]) & 15) for j in range(128)]
    scales = [int(blk[2112 + b]) for b in range(4)]
    return codes, scales


def test_mx_quantizer_crafted_blocks():
    s = 2.0 ** -3
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    b0 = [g * s for g in grid] + [-g * s for g in grid] + [6 * s] * 16          # on the grid, amax 6s
    b1 = [x * s for x in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0)] + [-0.2 * s, -0.25 * s] + [4 * s] * 22
    b2 = [0.0] * 32                                                              # all zero
    b3 = [3.0e38] + [1.0e-30] + [0.0] * 30                                       # extreme magnitudes
    codes, scales = _one_token(np.array(b0 + b1 + b2 + b3))
    # block 0: amax = 6 s = 0.75 -> E = floor(log2 0.75) - 2 = -3, lossless
    assert scales[0] == 127 - 3
    assert [brute.e2m1(c) for c in codes[:32]] == [g for g in grid] + [-g for g in grid] + [6.0] * 16
    # block 1: amax = 7 s = 0.875 -> E = floor(log2 0.875) - 2 = -3; ties go to the even code, 7 saturates to 6
    assert scales[1] == 127 - 3
    assert [brute.e2m1(c) for c in codes[32:40]] == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
    assert codes[40] == 8 and codes[41] == 8  # -0.2 and -0.25 round to -0 (sign kept)
    # block 2: all zero -> E = -127, zero codes
    assert scales[2] == 0 and codes[64:96] == [0] * 32
    # block 3: amax = bf16(3e38) -> E = 127 - 2 = 125; the tiny value flushes to 0
    assert scales[3] == 127 + 125
    assert brute.e2m1(codes[96]) * 2.0 ** 125 == pytest.approx(float(_bf16_value(3.0e38)), rel=0.2)
    for b, blk in enumerate((b0, b1, b2, b3)):
        want, e = brute.mx_quant_block(np.array([_bf16_value(x) for x in blk], np.float32))
        assert codes[32 * b:32 * b + 32] == want and scales[b] == e


def _bf16_value(x):
    return float((np.array([_bf16([x])[0]], np.uint32) << 16).view(np.float32)[0])


@pytest.fixture(scope="module")
def small():
    wl = make_workload(0, ctx=[1, 17, 145, 170, 230], Hq=4, Hkv=1, seed=61)
    hi = host_inputs(wl)
    return wl, hi, mx_cache(wl, hi)


def test_mx_blocks_hold_mxfp4_of_rotated_keys_and_values(small):
    wl, hi, cache = small
    for b in range(wl.B):
        for p in sorted({0, int(wl.ctx[b]) // 2, int(wl.ctx[b]) - 1}):
            k = oracle.bf16_to_f32(hi.k[hi.offsets[b] + p])[0]
            v = oracle.bf16_to_f32(hi.v[hi.offsets[b] + p])[0]
            kr = (brute.fwht_f32_recursive(k) * brute.inv_sqrt128_f32()).astype(np.float32)
            blk = cache.pages[wl.page_table[b, p // 16], 0]
            t = p % 16
            for blkno in range(4):
                kc, ke = brute.mx_quant_block(kr[32 * blkno:32 * blkno + 32])
                vc, ve = brute.mx_quant_block(v[32 * blkno:32 * blkno + 32])
                got_k = [(int(blk[64 * t + (32 * blkno + j) // 2]) >> (4 * (j % 2))) & 15 for j in range(32)]
                got_v = [(int(blk[1024 + 8 * (32 * blkno + j) + t // 2]) >> (4 * (t % 2))) & 15 for j in range(32)]
                assert got_k == kc and int(blk[2048 + 4 * t + blkno]) == ke
                assert got_v == vc and int(blk[2112 + 4 * t + blkno]) == ve


def test_mx_dequantization_error_bound(small):
    """|x^ - x| <= 2^E inside [-6, 6] 2^E (half the largest grid gap), and the
    storage is 4.25 bits per element (the page block keeps its size)."""
    wl, hi, cache = small
    assert cache.pages.shape[2] * 8 / (16 * 2 * 128) == 4.25
    b = 4
    for p in range(0, int(wl.ctx[b]), 7):
        v = oracle.bf16_to_f32(hi.v[hi.offsets[b] + p])[0]
        _, vv = brute.unpack_mx_block(cache.pages[wl.page_table[b, p // 16], 0])
        blk = cache.pages[wl.page_table[b, p // 16], 0]
        for blkno in range(4):
            E = int(blk[2112 + 4 * (p % 16) + blkno]) - 127
            err = np.abs(vv[p % 16, 32 * blkno:32 * blkno + 32] - v[32 * blkno:32 * blkno + 32])
            inside = np.abs(v[32 * blkno:32 * blkno + 32]) <= 6 * 2.0 ** E
            assert (err[inside] <= 2.0 ** E).all() and (err <= 2 * 2.0 ** E).all()


def test_mx_side_rows_and_appends(small):
    wl, hi, cache = small
    ref = oracle_cache(wl, hi)
    assert np.array_equal(cache.side_codes, ref.side_codes)
    assert np.array_equal(cache.side_scales, ref.side_scales)
    step = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots)
    for p in range(int(wl.ctx.max())):
        live = np.nonzero(wl.ctx > p)[0]
        rows = hi.offsets[live] + p
        oracle.mx_append(step, hi.k[rows], hi.v[rows], np.full(len(live), p, np.int32), wl.slots[live],
                         wl.page_table[live])
    assert np.array_equal(step.pages, cache.pages)


def test_mx_decode_matches_brute_force(small):
    wl, hi, cache = small
    out, lse = oracle.mx_decode(cache, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    sl = float(oracle.scale_log2(SCALE))
    for b in range(wl.B):
        for h in (0, 3):
            o, l = brute.mx_decode_one(cache.pages, cache.side_codes, cache.side_scales, hi.q[b, h],
                                       int(wl.ctx[b]), wl.slots[b], 0, wl.page_table[b], sl)
            assert np.abs(out[b, h] - o).max() < 1e-9
            assert abs(lse[b, h] - l) < 1e-9


def test_mx_all_protected_equals_kv4rl():
    wl = make_workload(0, ctx=[1, 30, 144], Hq=4, Hkv=1, seed=62)
    hi = host_inputs(wl)
    o1, l1 = oracle.mx_decode(mx_cache(wl, hi), hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table,
                              wl.Hq, SCALE)
    o2, l2, _ = oracle.decode(oracle_cache(wl, hi), hi.q, wl.ctx.astype(np.int32), wl.slots,
                              wl.page_table, wl.Hq, SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_mx_unprotected_is_softmax_over_dequantized_rows():
    """s = w = 0: one region; out = FP64 softmax of bf16(q_rot) . k^ over exactly
    dequantized MXFP4 rows (FP32 weights differ by rounding only)."""
    wl = make_workload(0, ctx=[5, 40, 97], Hq=4, Hkv=1, seed=63)
    hi = host_inputs(wl)
    cache = mx_cache(wl, hi, sink=0, window=0)
    out, lse = oracle.mx_decode(cache, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    for b in range(wl.B):
        for h in (0, 2):
            q = oracle.bf16_to_f32(hi.q[b, h])
            r = (brute.fwht_f32_recursive(q) * brute.inv_sqrt128_f32()).astype(np.float32)
            qb = np.array([brute.rnbf16(float(x)) for x in r])
            ks, vs = [], []
            for p in range(int(wl.ctx[b])):
                kk, vv = brute.unpack_mx_block(cache.pages[wl.page_table[b, p // 16], 0])
                ks.append(kk[p % 16])
                vs.append(vv[p % 16])
            z = SCALE * LOG2E * (np.array(ks) @ qb)
            e = np.exp2(z - z.max())
            assert np.abs(out[b, h] - (e[:, None] * np.array(vs)).sum(0) / e.sum()).max() < 1e-4
            assert abs(lse[b, h] - math.log(2) * (z.max() + math.log2(e.sum()))) < 1e-4
