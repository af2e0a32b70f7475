"""Pins of the oracle's cache writers: storage accounting, layout against an
independent unpacker, the sink/ring side rows, no INT4 rewrite on eviction."""
import json
import os

import numpy as np

import oracle
from oracle import brute
from synth import make_workload
from tests.wl import host_inputs, oracle_cache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_storage_is_4_25_bits_per_element():
    spec = json.load(open(os.path.join(GOLDEN, "kv4rl_budget.json")))
    # one group: 128 four-bit codes + FP16 delta + FP16 offset
    group_bits = spec["group_elements"] * spec["code_bits"] + 16 + 16
    assert group_bits / spec["group_elements"] == spec["bits_per_element"]
    cache = oracle.Cache(num_pages=3, Hkv=2, max_slots=1)
    positions = 3 * 16
    elements = positions * 2 * 2 * 128  # K and V, 2 kv-heads
    assert cache.pages.nbytes * 8 / elements == spec["bits_per_element"]
    assert cache.side_codes.shape[2] == spec["sink_positions"] + spec["recent_positions"]
    assert spec["protected_budget"] == cache.side_codes.shape[2]


def test_kv_bytes_formula_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "kv_size_example.json")))
    per_token = 2 * ex["layers"] * ex["kv_heads"] * ex["head_dim"] * ex["bytes_per_element"]
    assert per_token == ex["bytes_per_token"]
    assert per_token * ex["context"] == ex["bytes_per_request_gib"] * 2 ** 30
    assert per_token * ex["context"] * ex["requests"] == ex["bytes_all_requests_gib"] * 2 ** 30
    # the same accounting at 4.25 bits per element (one block row per page slot)
    block_row = oracle.BLOCK // oracle.PAGE  # bytes per (position, kv-head), K and V
    assert ex["layers"] * ex["kv_heads"] * block_row == per_token * 4.25 / 16


def test_pages_hold_quantized_rotated_keys_and_values():
    wl = make_workload(0)
    hi = host_inputs(wl)
    cache = oracle_cache(wl, hi)
    for b in range(wl.B):
        for p in (0, 15, 16, 17, int(wl.ctx[b]) - 2, int(wl.ctx[b]) - 1):
            k = oracle.bf16_to_f32(hi.k[hi.offsets[b] + p])   # [Hkv][128]
            v = oracle.bf16_to_f32(hi.v[hi.offsets[b] + p])
            kr = (brute.fwht_f32_recursive(k) * brute.inv_sqrt128_f32()).astype(np.float32)
            kc, kd, km = oracle.quant_int4(kr)
            vc, vd, vm = oracle.quant_int4(v)
            for g in range(wl.Hkv):
                blk = cache.pages[wl.page_table[b, p // 16], g]
                ukc, uvc, ukd, ukm, uvd, uvm = brute.unpack_block(blk)
                t = p % 16
                assert np.array_equal(ukc[t], kc[g]) and np.array_equal(uvc[t], vc[g])
                assert np.float16(ukd[t]) == kd[g].view(np.float16)
                assert np.float16(ukm[t]) == km[g].view(np.float16)
                assert np.float16(uvd[t]) == vd[g].view(np.float16)
                assert np.float16(uvm[t]) == vm[g].view(np.float16)


def _side_row(p):
    return p if p < 16 else 16 + p % 128


def test_ring_invariant_and_no_int4_rewrite_on_eviction():
    wl = make_workload(0, ctx=[300])
    hi = host_inputs(wl)
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots)
    L = int(wl.ctx[0])
    for p in range(L):
        before_pages = cache.pages.copy()
        before_side = cache.side_codes.copy()
        ka, va = hi.at([p])
        oracle.append(cache, ka, va, np.array([p], np.int32), wl.slots, wl.page_table)
        # only position p's bytes change in the INT4 pool ...
        changed = np.argwhere(before_pages != cache.pages)
        phys = wl.page_table[0, p // 16]
        t = p % 16
        for page, g, byte in changed:
            assert page == phys
            ok = (64 * t <= byte < 64 * t + 64) or (1024 <= byte < 2048 and (byte - 1024) % 8 == t // 2) \
                or (2048 + 4 * t <= byte < 2048 + 4 * t + 4) or (2112 + 4 * t <= byte < 2112 + 4 * t + 4)
            assert ok, (p, byte)
        # ... and only its own side row (the evicted position's INT4 entry stays)
        rows = np.unique(np.argwhere(before_side != cache.side_codes)[:, 2])
        assert set(rows.tolist()) <= {_side_row(p)}
    # after all appends: sinks 0..15 and the last 128 positions are in their rows
    for p in list(range(16)) + list(range(L - 128, L)):
        k = oracle.bf16_to_f32(hi.k[p])
        v = oracle.bf16_to_f32(hi.v[p])
        kr = (brute.fwht_f32_recursive(k) * brute.inv_sqrt128_f32()).astype(np.float32)
        k8, ks = oracle.quant_int8(kr)
        v8, vs = oracle.quant_int8(v)
        r = _side_row(p)
        assert np.array_equal(cache.side_codes[0, :, r, 0], k8)
        assert np.array_equal(cache.side_codes[0, :, r, 1], v8)
        assert np.array_equal(cache.side_scales[0, :, r, 0], ks)
        assert np.array_equal(cache.side_scales[0, :, r, 1], vs)


def test_prefill_in_chunks_equals_prefill_at_once():
    wl = make_workload(0)
    hi = host_inputs(wl)
    whole = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots)
    k, v, cu = hi.prefix(wl.ctx)
    oracle.prefill(whole, k, v, cu, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    parts = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots)
    first = wl.ctx // 3
    k1, v1, cu1 = hi.prefix(first)
    oracle.prefill(parts, k1, v1, cu1, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    rows = np.concatenate([np.arange(hi.offsets[b] + first[b], hi.offsets[b + 1]) for b in range(wl.B)])
    cu2 = np.zeros(wl.B + 1, np.int32)
    cu2[1:] = np.cumsum(wl.ctx - first)
    oracle.prefill(parts, hi.k[rows], hi.v[rows], cu2, first.astype(np.int32), wl.slots,
                   wl.page_table)
    assert np.array_equal(whole.pages, parts.pages)
    assert np.array_equal(whole.side_codes, parts.side_codes)
    assert np.array_equal(whole.side_scales, parts.side_scales)
