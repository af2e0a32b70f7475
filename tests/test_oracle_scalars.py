"""Pins of the oracle's scalar rules against things other than itself:
IEEE reference conversions, the Sylvester matrix, brute-force argmin
quantizers, error bounds, and high-precision exp2."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------- conversions --

def _dense_f32_sample():
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x7FFF, 0x8000, 0x8001, 0xFFFF],
                    dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    rnd = RNG.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, rnd])
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def test_f16_rne_matches_numpy():
    x = _dense_f32_sample()
    ours = oracle.f32_to_f16(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_to_f32_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_rne_matches_torch():
    x = _dense_f32_sample()
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# -------------------------------------------------------------- Hadamard --

def test_fwht_columns_are_sylvester():
    # FWHT of a basis vector has one non-zero term per output: exact.
    eye = np.eye(128, dtype=np.float32)
    cols = oracle.fwht(eye)
    s = np.float32(brute.inv_sqrt128_f32())
    assert np.array_equal(cols, (brute.sylvester(128) * s).astype(np.float32))


def test_hadamard_orthonormal_and_score_invariance():
    h = brute.sylvester(128)
    assert np.array_equal(h @ h.T, 128 * np.eye(128))  # exact in integers
    hn = h / math.sqrt(128)
    assert np.abs(hn @ hn.T - np.eye(128)).max() < 1e-15
    q = RNG.standard_normal((4, 128))
    k = RNG.standard_normal((9, 128))
    # row vectors: (q H)(k H)^T = q H H^T k^T = q k^T
    lhs = (q @ hn) @ (k @ hn).T
    assert np.abs(lhs - q @ k.T).max() <= 1e-12 * np.abs(q @ k.T).max() + 1e-12


def test_fwht_fp32_close_to_fp64_and_stage_order():
    x = (RNG.standard_normal((64, 128)) * RNG.choice([1, 20], (64, 128))).astype(np.float32)
    got = oracle.fwht(x).astype(np.float64)
    exact = x.astype(np.float64) @ (brute.sylvester(128) / math.sqrt(128))
    # 7 rounded stages plus one rounded scaling, each within 2^-24 relative
    bound = 8 * 2.0 ** -24 * (np.abs(x).astype(np.float64).sum(1, keepdims=True) / math.sqrt(128))
    assert (np.abs(got - exact) <= bound + 2.0 ** -24 * np.abs(exact)).all()
    # The stride order 1, 2, ..., 64 fixes the FP32 sum tree: the recursive
    # Sylvester evaluation (outermost split = stride 64, applied last) has
    # exactly that tree.
    ref = (brute.fwht_f32_recursive(x) * brute.inv_sqrt128_f32()).astype(np.float32)
    assert np.array_equal(oracle.fwht(x), ref)


def test_fwht_stage_order_explicit_tree():
    # element 0 = (((((((x0+x1)+(x2+x3))+...) pairwise, strides 1 then 2 then ...
    x = (RNG.standard_normal(128) * 1000).astype(np.float32)
    level = x.copy()
    while level.size > 1:
        level = (level[0::2] + level[1::2]).astype(np.float32)
    want = np.float32(level[0] * brute.inv_sqrt128_f32())
    assert oracle.fwht(x)[0] == want


def test_inv_sqrt128_constant():
    assert np.float32(brute.inv_sqrt128_f32()).view(np.uint32) == 0x3DB504F3


# ------------------------------------------------------------ quantizers --

def _vectors(n=400):
    x = RNG.standard_normal((n, 128)).astype(np.float32)
    x[: n // 4] *= 20
    x[n // 4: n // 2] += RNG.standard_normal((n // 4, 1)).astype(np.float32) * 50
    return x


def test_int4_codes_are_nearest_grid_points():
    x = _vectors()
    codes, d16, m16 = oracle.quant_int4(x)
    d = d16.view(np.float16).astype(np.float64)[:, None]
    m = m16.view(np.float16).astype(np.float64)[:, None]
    xs = x.astype(np.float64)
    # Delta and m follow the stated rule with an independent RNE (numpy)
    mn, mx = x.min(1), x.max(1)
    assert np.array_equal(d16, ((mx - mn).astype(np.float32) / np.float32(15)).astype(np.float16).view(np.uint16))
    assert np.array_equal(m16, mn.astype(np.float16).view(np.uint16))
    # every code, ties included, equals the exact-rational rule
    # (rn32(x - m), rn32(/ delta), round half to even, clamp)
    want = np.array([brute.quant_int4_exact(row)[0] for row in x], np.uint8)
    assert np.array_equal(codes, want)
    # and it is a nearest grid point: its distance exceeds the best one by at
    # most the FP32 rounding of x - m and of the quotient
    grid = d * np.arange(16)[None, :] + m                    # [n, 16]
    dist = np.abs(xs[:, :, None] - grid[:, None, :])        # [n, 128, 16]
    mine = np.take_along_axis(dist, codes[..., None].astype(np.int64), -1)[..., 0]
    slack = 2.0 ** -22 * (np.abs(xs) + np.abs(m) + 16 * d)
    assert (mine <= dist.min(-1) + slack).all()
    # dequantization error bound for elements inside the grid
    xhat = d * codes + m
    inside = (xs >= m) & (xs <= m + 15 * d)
    err = np.abs(xs - xhat)
    bound = np.broadcast_to(d / 2, err.shape) + 1e-6 * np.maximum(np.abs(xs), 1)
    assert (err <= bound)[inside].all()
    # clamped extremes: within delta/2 + |m - min| + 15 |delta - range/15|
    slack = d / 2 + np.abs(m - mn[:, None]) + 15 * np.abs(d - ((mx - mn) / 15.0)[:, None]) + 1e-5
    assert (err <= slack).all()


def test_int4_constant_and_grid_exact_vectors():
    c = np.full((3, 128), 0.7, np.float32)
    codes, d16, m16 = oracle.quant_int4(c)
    assert (codes == 0).all() and (d16 == 0).all()
    # grid-exact input: x = m + delta*c with FP16-exact delta, m is lossless
    rng = np.random.default_rng(7)
    want = rng.integers(0, 16, (5, 128))
    want[:, 0], want[:, 1] = 0, 15
    delta, m = np.float32(0.125), np.float32(-1.5)
    x = (m + delta * want).astype(np.float32)
    codes, d16, m16 = oracle.quant_int4(x)
    assert np.array_equal(codes, want)
    assert (d16.view(np.float16) == np.float16(0.125)).all()


def test_int8_symmetric_nearest_and_odd():
    x = _vectors()
    codes, s16 = oracle.quant_int8(x)
    s = s16.view(np.float16).astype(np.float64)[:, None]
    a = np.abs(x).max(1)
    assert np.array_equal(s16, (a / np.float32(127)).astype(np.float16).view(np.uint16))
    q = x.astype(np.float64) / s
    # every code, ties included, equals the exact-rational rule
    want = np.array([brute.quant_int8_exact(row)[0] for row in x], np.int8)
    assert np.array_equal(codes, want)
    # and it is the nearest integer of the FP64 quotient, a tie (exactly
    # representable there) going to the even code
    assert np.array_equal(codes, np.clip(np.rint(q), -127, 127).astype(np.int8))
    err = np.abs(x - s * codes)
    inside = np.abs(q) <= 127
    assert (err[inside] <= (np.broadcast_to(s, err.shape)[inside] / 2) * (1 + 1e-6)).all()
    neg_codes, _ = oracle.quant_int8(-x)
    assert np.array_equal(neg_codes, -codes)
    z, zs = oracle.quant_int8(np.zeros((2, 128), np.float32))
    assert (z == 0).all() and (zs == 0).all()


def test_query_quantizer_fp32_scale():
    x = _vectors(100)
    codes, s, sm = oracle.quant_query(x)
    a = np.abs(x).max(1)
    assert np.array_equal(s, (a / np.float32(127)).astype(np.float32))
    assert np.array_equal(sm, codes.astype(np.int64).sum(1))
    # brute force with exact division rounding
    for i in range(0, 100, 9):
        want = [min(127, max(-127, brute.rint_even(brute.f32_div(float(v), float(s[i])))))
                for v in x[i]]
        assert list(codes[i]) == want
    # the largest magnitude maps to +-127
    assert (np.abs(codes).max(1) == 127).all()


# ------------------------------------------------------------------ exp2 --

def test_exp2s_coefficients_exact():
    ours = oracle.exp2s_coeffs()
    assert list(ours) == [np.float32(c) for c in brute.exp2_coeffs_exact()]


def test_exp2s_accuracy_and_cutoff():
    y = np.concatenate([np.linspace(-125, 0, 3_000_001, dtype=np.float32),
                        -RNG.random(1_000_000).astype(np.float32) * 125])
    e = oracle.exp2s(y).astype(np.float64)
    ref = np.exp2(y.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert (np.abs(e - ref) <= 2 * ulp).all()
    assert oracle.exp2s(np.array([0.0], np.float32))[0] == 1.0
    assert (oracle.exp2s(np.array([-125.0001, -126, -1e30, -np.inf], np.float32)) == 0).all()


def test_exp2s_matches_exact_rational_evaluation():
    y = np.concatenate([-RNG.random(1500) * 20, -RNG.random(500) * 125]).astype(np.float32)
    ours = oracle.exp2s(y)
    want = np.array([brute.exp2s(float(v)) for v in y], np.float32)
    assert np.array_equal(ours, want)


def test_scale_log2():
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    log2e = float(1 / Decimal(2).ln())  # correctly rounded double of log2(e)
    s = np.float32(1.0 / math.sqrt(128))
    assert oracle.scale_log2(float(s)) == np.float32(float(s) * log2e)
