"""Exact pins of the cache quantizers at and next to rounding ties.

The INT4 and INT8 codes are decided by FP32 arithmetic (a subtraction, an IEEE
division, round-half-to-even), and near a half-integer quotient only that
exact sequence gives the right code.  Here every step is redone with exact
rational arithmetic and an explicit round-to-nearest-even to binary32
(oracle/brute.py), on vectors crafted so that most elements sit on a tie or a
few FP32 ulps from one (x = m + (c + 1/2)*delta +- k ulp; x = +-(c + 1/2)*s
+- k ulp), including FP16-subnormal deltas and scales, offsets that make the
subtraction round, and values just inside the clamp limits.  The oracle must
agree on every code and every FP16 metadata bit pattern (KV4-RL pages,
paper.rainbus.top summary, "分组仿射 KV 量化" and "方法步骤详情" steps 2-3).

Each test also evaluates plausible wrong orders of the same arithmetic
(reciprocal multiply, a fused multiply-add, a split division, division in
FP64, an unrounded subtraction) and requires the crafted set to tell each
of them apart from the rule, so that the pin has teeth.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute

HD = 128
RNG = np.random.default_rng(20261202)


def _f32(x) -> np.float32:
    return np.float32(brute.rn32(Fraction(x)))


def _step_ulps(x: np.float32, k: int) -> np.float32:
    d = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
    for _ in range(abs(k)):
        x = np.nextafter(x, d)
    return np.float32(x)


# ------------------------------------------------------------------ INT4 --

def _int4_rule(x, mn, mx):
    """Codes, delta and m of one vector by exact rational steps (min and max
    of the crafted vector are mn and mx)."""
    assert float(min(x)) == float(mn) and float(max(x)) == float(mx)
    return brute.quant_int4_exact(x)


def _int4_case(kind: str):
    """One crafted vector: its min and max first, then 126 elements placed on
    or next to the half-way points between grid codes."""
    if kind == "subnormal":      # FP16-subnormal delta, tiny offset
        mn = _f32(-RNG.uniform(0, 3e-5))
        rng_ = RNG.uniform(1e-5, 8e-4)
    elif kind == "straddle":     # negative min, positive max: x - m rounds in FP32
        mn = _f32(-RNG.uniform(200, 2000) * (1 + RNG.random()))
        rng_ = -float(mn) * RNG.uniform(1.5, 2.5)
    elif kind == "offset":       # large positive offset, small range
        mn = _f32(RNG.uniform(100, 3000))
        rng_ = RNG.uniform(0.05, 40)
    else:                        # ordinary magnitudes
        mn = _f32(-RNG.uniform(0.01, 60))
        rng_ = RNG.uniform(0.01, 120)
    mx = _f32(Fraction(float(mn)) + Fraction(rng_))
    d = brute.rn16(Fraction(brute.f32_div(brute.f32_sub(float(mx), float(mn)), 15.0)))
    m = brute.rn16(Fraction(float(mn)))
    x = [mn, mx]
    while len(x) < HD:
        c = int(RNG.integers(-1, 16))  # -1 and 15: the clamp edges
        k = int(RNG.integers(-3, 4))
        v = _step_ulps(_f32(Fraction(m) + (Fraction(c) + Fraction(1, 2)) * Fraction(d)), k)
        x.append(v if mn <= v <= mx else (mn if RNG.random() < 0.5 else mx))
    x = np.array(x, np.float32)
    RNG.shuffle(x)
    return x, mn, mx


INT4_KINDS = ["plain"] * 70 + ["subnormal"] * 30 + ["straddle"] * 30 + ["offset"] * 30


@pytest.fixture(scope="module")
def int4_set():
    xs, want_c, want_d, want_m = [], [], [], []
    for kind in INT4_KINDS:
        x, mn, mx = _int4_case(kind)
        c, d, m = _int4_rule(x, mn, mx)
        xs.append(x)
        want_c.append(c)
        want_d.append(d)
        want_m.append(m)
    return (np.stack(xs), np.array(want_c, np.uint8), np.array(want_d, np.float64),
            np.array(want_m, np.float64))


def test_int4_codes_exact_at_ties(int4_set):
    x, want, d, m = int4_set
    assert x.size >= 10_000
    codes, d16, m16 = oracle.quant_int4(x)
    assert np.array_equal(d16.view(np.float16).astype(np.float64), d)
    assert np.array_equal(m16.view(np.float16).astype(np.float64), m)
    assert np.array_equal(codes, want)
    # the set really is made of ties: the exact quotient (x - m) / delta is
    # within a few FP32 ulps of a half-integer for most elements (a few
    # hundred ulps where a large offset makes x - m coarse), exactly on one
    # for some
    q = np.array([[float((Fraction(float(v)) - Fraction(float(mi))) / Fraction(float(di))) if di else 0.0
                   for v in row] for row, mi, di in zip(x, m, d)])
    dist = np.abs(np.abs(q - np.floor(q)) - 0.5)
    assert (dist < 1e-5).mean() > 0.6
    assert (dist < 1e-3).mean() > 0.8  # the rest: min, max and the clamp-edge fillers
    assert (dist == 0).sum() > 100
    assert (d16.view(np.float16) < np.float16(2 ** -14)).sum() >= 25  # FP16-subnormal deltas


def _int4_mutants(x, d, m):
    """Wrong orders of the same arithmetic, in numpy binary32 (IEEE RN)."""
    x = x.astype(np.float32)
    d32 = d.astype(np.float32)[:, None]
    m32 = m.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(1) / d32
        mut = {
            "reciprocal multiply": (x - m32) * inv,
            "fused multiply-add": np.array([[brute.f32_fma(float(v), float(iv), float(-mi * iv))
                                             for v in row] for row, iv, mi in zip(x, inv[:, 0], m32[:, 0])],
                                           np.float32),
            "split division": x / d32 - m32 / d32,
            "division in FP64": (x.astype(np.float64) - m[:, None]) / d[:, None],
            "unrounded subtraction": np.array([[float(brute.rn32((Fraction(float(v)) - Fraction(float(mi)))
                                                                 / Fraction(float(di)))) if di else 0.0
                                                for v in row] for row, mi, di in zip(x, m, d)]),
        }
    out = {}
    for name, q in mut.items():
        q = np.where(d[:, None] == 0, 0.0, np.nan_to_num(np.asarray(q, np.float64)))
        out[name] = np.clip(np.rint(q), 0, 15).astype(np.uint8)
    return out


def test_int4_tie_set_separates_wrong_arithmetic(int4_set):
    x, want, d, m = int4_set
    for name, codes in _int4_mutants(x, d, m).items():
        assert (codes != want).sum() > 0, f"the crafted set does not catch: {name}"


# ------------------------------------------------------------------ INT8 --

def _int8_rule(x):
    return brute.quant_int8_exact(x)


def _int8_case(kind: str):
    if kind == "subnormal":
        a = _f32(RNG.uniform(1e-4, 7.5e-3))
    elif kind == "large":
        a = _f32(RNG.uniform(1000, 60000))
    else:
        a = _f32(RNG.uniform(0.05, 200))
    s = brute.rn16(Fraction(brute.f32_div(float(a), 127.0)))
    x = [a if RNG.random() < 0.5 else -a]
    while len(x) < HD:
        c = int(RNG.integers(0, 127))
        k = int(RNG.integers(-3, 4))
        v = _step_ulps(_f32((Fraction(c) + Fraction(1, 2)) * Fraction(s)), k)
        v = v if RNG.random() < 0.5 else -v
        x.append(v if abs(v) <= a else x[0])
    x = np.array(x, np.float32)
    RNG.shuffle(x)
    return x


INT8_KINDS = ["plain"] * 90 + ["subnormal"] * 30 + ["large"] * 30


@pytest.fixture(scope="module")
def int8_set():
    xs, want, ss = [], [], []
    for kind in INT8_KINDS:
        x = _int8_case(kind)
        c, s = _int8_rule(x)
        xs.append(x)
        want.append(c)
        ss.append(s)
    return np.stack(xs), np.array(want, np.int8), np.array(ss, np.float64)


def test_int8_codes_exact_at_ties(int8_set):
    x, want, s = int8_set
    assert x.size >= 10_000
    codes, s16 = oracle.quant_int8(x)
    assert np.array_equal(s16.view(np.float16).astype(np.float64), s)
    assert np.array_equal(codes, want)
    q = np.array([[float(Fraction(float(v)) / Fraction(float(si))) for v in row] for row, si in zip(x, s)])
    dist = np.abs(np.abs(q - np.floor(q)) - 0.5)
    ulps = dist / np.spacing(np.abs(q).astype(np.float32)).astype(np.float64)
    assert (ulps <= 4).mean() > 0.9  # within 4 FP32 ulps of the quotient
    assert (dist == 0).sum() > 100
    assert (s16.view(np.float16) < np.float16(2 ** -14)).sum() >= 25  # FP16-subnormal scales
    # odd symmetry holds exactly at ties too (round half to even is symmetric)
    neg, _ = oracle.quant_int8(-x)
    assert np.array_equal(neg, -codes)


def test_int8_tie_set_separates_wrong_arithmetic(int8_set):
    x, want, s = int8_set
    s32 = s.astype(np.float32)[:, None]
    # (Division in FP64 is no mistake here: with an FP16 scale of at most 11
    # significant bits, x / s is either exactly a half-integer or at least
    # about one FP32 ulp away from it, so both divisions give the same code;
    # checked below rather than required to differ.)
    with np.errstate(divide="ignore"):
        mut = {"reciprocal multiply": x * (np.float32(1) / s32),
               "round half away from zero": np.trunc(x / s32 + np.copysign(np.float32(0.5), x))}
        same = np.clip(np.rint(x.astype(np.float64) / s[:, None]), -127, 127).astype(np.int8)
    assert np.array_equal(same, want)
    for name, q in mut.items():
        codes = np.clip(np.rint(np.asarray(q, np.float64)), -127, 127).astype(np.int8)
        assert (codes != want).sum() > 0, f"the crafted set does not catch: {name}"
