"""Pins of the oracle's re-prefill (chunked-prefill) attention over the KV4-RL
cache (KV4-RL pages, partial rollout: carried prefixes re-prefilled after a
weight update).  Reading: after a chunk's K/V are written, token p attends
[0, p] under the protected set of the cache as it stands (sinks, and the
recent window [E - w, E) of the cache ending at E); a one-token chunk is a
decode step."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import make_workload
from tests.wl import host_inputs

SCALE = 1.0 / math.sqrt(128)
LOG2E = 1.0 / math.log(2.0)


def _full_cache(wl, hi, sink=16, window=128):
    cache = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    k, v, cu = hi.prefix(wl.ctx)
    oracle.prefill(cache, k, v, cu, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    return cache


def _chunk_queries(wl, hi, start, n, layer_seed=5):
    """Seeded BF16 queries for the chunk tokens: [T][Hq][128]."""
    rng = np.random.default_rng(layer_seed)
    T = int(np.sum(n))
    q = rng.standard_normal((T, wl.Hq, 128)).astype(np.float32)
    import torch
    return torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_one_token_chunks_equal_decode():
    wl = make_workload(0, ctx=[1, 17, 145, 170, 300], Hq=4, Hkv=1, seed=81)
    hi = host_inputs(wl)
    cache = _full_cache(wl, hi)
    cu = np.arange(wl.B + 1, dtype=np.int32)
    out, lse, dbg = oracle.prefill_attention(cache, hi.q, cu, (wl.ctx - 1).astype(np.int32), wl.slots,
                                             wl.page_table, wl.Hq, SCALE, debug=True)
    o2, l2, d2 = oracle.decode(cache, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE,
                               debug=True)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    for key in d2:
        assert np.array_equal(dbg[key], d2[key]), key


@pytest.fixture(scope="module")
def chunk():
    # two sequences: chunks of 40 and 23 tokens ending at 230 and 60
    wl = make_workload(0, ctx=[230, 60], Hq=4, Hkv=1, seed=82)
    hi = host_inputs(wl)
    cache = _full_cache(wl, hi)
    n = np.array([40, 23], np.int32)
    start = (wl.ctx - n).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = _chunk_queries(wl, hi, start, n)
    return wl, hi, cache, n, start, cu, q


def test_last_token_of_a_chunk_is_a_decode_step(chunk):
    wl, hi, cache, n, start, cu, q = chunk
    out, lse, _ = oracle.prefill_attention(cache, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE)
    last = cu[1:] - 1
    o2, l2, _ = oracle.decode(cache, q[last], wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    assert np.array_equal(out[last], o2) and np.array_equal(lse[last], l2)


def test_prefill_attention_matches_brute_force(chunk):
    wl, hi, cache, n, start, cu, q = chunk
    out, lse, dbg = oracle.prefill_attention(cache, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE,
                                             debug=True)
    sl = float(oracle.scale_log2(SCALE))
    for s in range(wl.B):
        E = int(wl.ctx[s])
        for i in (0, int(n[s]) // 2, int(n[s]) - 1):
            t = int(cu[s]) + i
            L = int(start[s]) + i + 1
            for h in (0, 3):
                o, l, qk, pc, pv = brute.decode_one(cache.pages, cache.side_codes, cache.side_scales, wl.Hkv,
                                                    q[t, h], L, wl.slots[s], 0, wl.page_table[s], sl, E=E)
                assert sorted(qk) == list(range(L))
                assert np.abs(out[t, h] - o).max() < 1e-9 and abs(lse[t, h] - l) < 1e-9
                for p, d in qk.items():
                    assert dbg["qk"][t, h, p] == d
                for p, c in pc.items():
                    assert dbg["pcode"][t, h, p] == c
                for j, acc in pv.items():
                    assert np.array_equal(dbg["pv"][t, h, j], acc)


def test_prefill_attention_is_causal(chunk):
    """Garbage in every cache entry of positions after p (page nibbles and
    metadata, side rows) leaves the first chunk token's output unchanged."""
    wl, hi, cache, n, start, cu, q = chunk
    out0, lse0, _ = oracle.prefill_attention(cache, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE)
    rng = np.random.default_rng(3)
    c2 = cache.copy()
    for s in range(wl.B):
        p0 = int(start[s])
        for p in range(p0 + 1, int(wl.ctx[s])):
            blk = c2.pages[wl.page_table[s, p // 16], 0]
            t = p % 16
            blk[64 * t:64 * t + 64] = rng.integers(0, 256, 64)
            blk[2048 + 4 * t:2052 + 4 * t] = rng.integers(0, 256, 4)
            blk[2112 + 4 * t:2116 + 4 * t] = rng.integers(0, 256, 4)
            nib = rng.integers(0, 16, 128).astype(np.uint8)
            keep = 0xF0 if t % 2 == 0 else 0x0F
            blk[1024 + t // 2:2048:8] = (blk[1024 + t // 2:2048:8] & keep) | (nib << (0 if t % 2 == 0 else 4))
            if p >= 16:
                row = 16 + p % 128
                c2.side_codes[wl.slots[s], 0, row] = rng.integers(-127, 128, (2, 128))
    out1, lse1, _ = oracle.prefill_attention(c2, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE)
    first = cu[:-1]
    assert np.array_equal(out0[first], out1[first]) and np.array_equal(lse0[first], lse1[first])


def test_prefill_attention_exact_pv_is_causal_softmax(chunk):
    """Exact-PV mode = FP64 softmax over [0, p]: protected positions (sinks,
    window of the cache) from the INT8 side rows, the rest from INT4."""
    wl, hi, cache, n, start, cu, q = chunk
    out, lse, _ = oracle.prefill_attention(cache, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE,
                                           pv_exact=True)
    for s in range(wl.B):
        E = int(wl.ctx[s])
        for i in (0, int(n[s]) - 5):
            t = int(cu[s]) + i
            L = int(start[s]) + i + 1
            prot = set(range(min(16, L))) | set(range(max(16, E - 128), L))
            for h in (1, 2):
                qc, s_q, _ = brute.query_codes(q[t, h])
                qhat = s_q * qc.astype(np.float64)
                z, vals = [], []
                for p in range(L):
                    if p in prot:
                        row = p if p < 16 else 16 + p % 128
                        sc = cache.side_scales[wl.slots[s], 0, row].view(np.float16).astype(np.float64)
                        kk = sc[0] * cache.side_codes[wl.slots[s], 0, row, 0].astype(np.float64)
                        vv = np.array([brute.rnbf16(sc[1] * float(c)) for c in cache.side_codes[wl.slots[s], 0, row, 1]])
                    else:
                        kc, vc, kd, km, vd, vm = brute.unpack_block(cache.pages[wl.page_table[s, p // 16], 0])
                        kk = kd[p % 16] * kc[p % 16] + km[p % 16]
                        vv = vd[p % 16] * vc[p % 16] + vm[p % 16]
                    z.append(SCALE * LOG2E * float(qhat @ kk))
                    vals.append(vv)
                z, vals = np.array(z), np.array(vals)
                e = np.exp2(z - z.max())
                assert np.abs(out[t, h] - (e[:, None] * vals).sum(0) / e.sum()).max() < 1e-4
                assert abs(lse[t, h] - math.log(2) * (z.max() + math.log2(e.sum()))) < 1e-4


def test_sampled_entry_equals_full(chunk):
    """The sampled entry point returns the full call's rows for the listed
    (token, head) pairs (the same arithmetic, the rest skipped)."""
    wl, hi, cache, n, start, cu, q = chunk
    out, lse, _ = oracle.prefill_attention(cache, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE)
    tokens = np.array([0, 5, 39, 40, 62], np.int64)
    heads = np.array([0, 3, 1, 2, 3], np.int64)
    o2, l2 = oracle.prefill_attention_sampled(cache, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE,
                                              tokens, heads)
    assert np.array_equal(o2, out[tokens, heads]) and np.array_equal(l2, lse[tokens, heads])
