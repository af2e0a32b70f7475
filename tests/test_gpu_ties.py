"""Cache writers at rounding ties on the GPU: value vectors crafted so that
many elements sit exactly on a half-way point of the INT4 grid (x - m a
half-integer multiple of delta) or of the INT8 grid (x a half-integer
multiple of s), or one BF16 ulp from one, go through kv4_append (every
position), kv4_prefill_quantize and the one-launch step; page blocks and side
rows must equal the oracle's byte for byte.  The oracle's quantizers are
pinned at such ties by exact rational arithmetic (tests/test_oracle_ties.py).

Values are BF16, so the crafted elements are half-way points that BF16 can
hold: deltas and scales that are small multiples of a power of two give exact
ties; other ranges give near-ties at BF16 spacing; a few vectors have
FP16-subnormal deltas or scales.  Keys are ordinary N(0,1) vectors (their
rotated values are not steerable), and the device quantizer that decides the
codes is one function for K and V (KV4-RL pages, paper.rainbus.top summary,
"分组仿射 KV 量化" and "方法步骤详情" steps 1-3)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from tests.gpu_util import SCALE, bf, i32
from tests.wl import HostInputs

pytestmark = pytest.mark.gpu

HD = 128


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _bf16_value(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _bf16_step(b: np.ndarray, k: np.ndarray) -> np.ndarray:
    """k BF16 ulps away (toward +inf for k > 0), for finite nonzero values."""
    v = b.astype(np.int64)
    sign = np.where(v & 0x8000, -1, 1)
    return (v + sign * k).astype(np.uint16)


def int4_tie_vector(rng) -> np.ndarray:
    kind = rng.integers(0, 4)
    if kind == 0:      # delta a power of two: every half-way point exact in BF16
        e = int(rng.integers(-9, 7))
        d = 2.0 ** e
        mn = d * int(rng.integers(-40, 40))
    elif kind == 1:    # delta = 3 * 2^e
        e = int(rng.integers(-9, 5))
        d = 3.0 * 2.0 ** e
        mn = 2.0 ** e * int(rng.integers(-40, 40))
    elif kind == 2:    # FP16-subnormal delta
        e = int(rng.integers(-22, -15))
        d = 2.0 ** e
        mn = d * int(rng.integers(-20, 20))
    else:              # an ordinary range: near-ties at BF16 spacing
        mn = float(-rng.uniform(0.05, 40))
        d = float(rng.uniform(0.01, 8))
    lo, hi = _bf16_bits(np.float32([mn, mn + 15 * d]))
    # the grid the quantizer will use (its own rounding, numpy RNE)
    mnv, mxv = _bf16_value(np.array([lo, hi]))
    dq = np.float32(np.float32(mxv - mnv) / np.float32(15)).astype(np.float16).astype(np.float64)
    mq = np.float32(mnv).astype(np.float16).astype(np.float64)
    c = rng.integers(0, 15, HD - 2)
    tie = _bf16_bits((mq + (c + 0.5) * dq).astype(np.float32))
    k = rng.choice([-1, 0, 0, 0, 1], HD - 2)
    body = np.where(tie & 0x7FFF, _bf16_step(tie, k), tie)
    vals = _bf16_value(body)
    body = np.where((vals >= mnv) & (vals <= mxv), body, lo)
    x = np.concatenate([[lo, hi], body]).astype(np.uint16)
    rng.shuffle(x)
    return x


def int8_tie_vector(rng) -> np.ndarray:
    kind = rng.integers(0, 3)
    if kind == 0:      # s a power of two
        s = 2.0 ** int(rng.integers(-8, 6))
    elif kind == 1:    # FP16-subnormal s
        s = 2.0 ** int(rng.integers(-22, -15))
    else:
        s = float(rng.uniform(0.002, 1.0))
    a = _bf16_bits(np.float32([127 * s]))
    av = float(_bf16_value(a)[0])
    sq = np.float32(np.float32(av) / np.float32(127)).astype(np.float16).astype(np.float64)
    c = rng.integers(0, 127, HD - 1)
    tie = _bf16_bits(((c + 0.5) * sq * rng.choice([-1.0, 1.0], HD - 1)).astype(np.float32))
    k = rng.choice([-1, 0, 0, 0, 1], HD - 1)
    body = np.where(tie & 0x7FFF, _bf16_step(tie, k), tie)
    body = np.where(np.abs(_bf16_value(body)) <= av, body, a[0])
    x = np.concatenate([a, body]).astype(np.uint16)
    rng.shuffle(x)
    return x


def crafted_inputs(ctx, Hkv, Hq, seed):
    """Keys N(0,1) in BF16; values crafted per (position, kv-head): INT8-tie
    vectors at odd positions that end in a side row (sinks, last 128), INT4-tie
    vectors everywhere else."""
    rng = np.random.default_rng(seed)
    n = int(np.sum(ctx))
    k = _bf16_bits(rng.standard_normal((n, Hkv, HD)).astype(np.float32))
    q = _bf16_bits(rng.standard_normal((len(ctx), Hq, HD)).astype(np.float32))
    v = np.empty((n, Hkv, HD), np.uint16)
    off = np.zeros(len(ctx) + 1, np.int64)
    off[1:] = np.cumsum(ctx)
    for b, L in enumerate(ctx):
        for p in range(L):
            side = p < 16 or p >= L - 128
            for g in range(Hkv):
                v[off[b] + p, g] = int8_tie_vector(rng) if (side and p % 2) else int4_tie_vector(rng)
    return HostInputs(k, v, q, off)


def tie_share(v_bits):
    """Share of elements on or within one BF16 ulp of an INT4 half-way point
    (FP64 check on the quantizer's own grid)."""
    x = _bf16_value(v_bits.reshape(-1, HD)).astype(np.float64)
    mn, mx = x.min(1), x.max(1)
    d = ((mx - mn).astype(np.float32) / np.float32(15)).astype(np.float16).astype(np.float64)
    m = mn.astype(np.float16).astype(np.float64)
    ok = d > 0
    q = (x[ok] - m[ok, None]) / d[ok, None]
    frac = np.abs(q - np.floor(q) - 0.5)
    return float((frac == 0).mean()), float((frac < 0.02).mean())


CASES = [("ties_a", [40, 150, 201, 333], 2, 8, 7), ("ties_b", [17, 145, 160, 288, 300, 1000], 1, 4, 8)]


@pytest.mark.parametrize("name,ctx,Hkv,Hq,seed", CASES)
def test_writers_at_ties_equal_oracle(name, ctx, Hkv, Hq, seed):
    _say(f"[ties] {name}: ctx {ctx} Hkv {Hkv}")
    dev = torch.device("cuda")
    ctx = np.array(ctx, np.int64)
    B = len(ctx)
    hi = crafted_inputs(ctx, Hkv, Hq, seed)
    exact, near = tie_share(hi.v)
    assert exact > 0.15 and near > 0.3, (exact, near)
    pages_per = (ctx + 15) // 16
    W = int(pages_per.max())
    num_pages = int(pages_per.sum()) + 5
    perm = np.random.default_rng(seed + 100).permutation(num_pages).astype(np.int32)
    table = np.zeros((B, W), np.int32)
    o = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[o:o + n]
        o += n
    slots = np.random.default_rng(seed + 200).permutation(B).astype(np.int32)
    lead = ctx - 1
    k_lead, v_lead, cu = hi.prefix(lead)
    ka, va = hi.at(lead)

    # oracle: re-prefill of [0, L-1), then this step's append
    ref = oracle.Cache(num_pages, Hkv, B)
    oracle.prefill(ref, k_lead, v_lead, cu, np.zeros(B, np.int32), slots, table)
    oracle.append(ref, ka, va, lead.astype(np.int32), slots, table)
    ref_out, ref_lse, _ = oracle.decode(ref, hi.q, ctx.astype(np.int32), slots, table, Hq, SCALE)

    t_table, t_slots = i32(table, dev), i32(slots, dev)

    def check(cache, how):
        torch.cuda.synchronize()
        assert np.array_equal(cache.pages.cpu().numpy(), ref.pages), f"{how}: page bytes differ"
        assert np.array_equal(cache.side_codes.cpu().numpy(), ref.side_codes), f"{how}: side codes differ"
        assert np.array_equal(cache.side_scales.cpu().numpy().view(np.uint16), ref.side_scales), \
            f"{how}: side scales differ"

    # 1. every position by kv4_append, in position order
    a = kv4.Kv4Cache.zeros(num_pages, Hkv, B, dev)
    for p in range(int(ctx.max())):
        rows = np.nonzero(ctx > p)[0]
        kp, vp = hi.at(np.where(ctx > p, p, 0))
        kv4.append(a, bf(kp[rows], dev), bf(vp[rows], dev), i32(np.full(len(rows), p), dev),
                   i32(slots[rows], dev), i32(table[rows], dev))
    check(a, "appends")
    # 2. re-prefill of [0, L-1), then kv4_append
    b_ = kv4.Kv4Cache.zeros(num_pages, Hkv, B, dev)
    kv4.prefill_quantize(b_, bf(k_lead, dev), bf(v_lead, dev), i32(cu, dev), i32(np.zeros(B), dev), t_slots,
                         t_table, int(lead.max()))
    kv4.append(b_, bf(ka, dev), bf(va, dev), i32(lead, dev), t_slots, t_table)
    check(b_, "re-prefill + append")
    # 3. re-prefill, then the one-launch step (the protected workgroups write the token)
    c_ = kv4.Kv4Cache.zeros(num_pages, Hkv, B, dev)
    kv4.prefill_quantize(c_, bf(k_lead, dev), bf(v_lead, dev), i32(cu, dev), i32(np.zeros(B), dev), t_slots,
                         t_table, int(lead.max()))
    out, lse = kv4.append_decode_attention(c_, bf(ka, dev), bf(va, dev), i32(lead, dev), bf(hi.q, dev),
                                           i32(ctx, dev), t_slots, t_table, int(ctx.max()), SCALE)
    check(c_, "one-launch step")
    assert np.abs(out.cpu().numpy() - ref_out).max() <= 2e-3
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-4
    _say(f"[ties] {name}: exact ties {exact:.1%}, within 0.02 of a tie {near:.1%}; bytes equal on 3 paths")
