"""Brute-force cross-check of the oracle on tiny inputs (test infrastructure).

Independent of oracle/kv4_oracle.c: it reads the packed cache with its own
unpacker written from the layout description, evaluates every FP32 step the
rules name with exact rational arithmetic followed by an explicit
round-to-nearest-even to binary32, gets the Hadamard rotation from the
recursive Sylvester construction H_2n = [[H, H], [H, -H]], and does every
tolerance-level sum in FP64.  Slow by design: a few sequences, a few hundred
positions.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

HD, PAGE, SINK, WINDOW = 128, 16, 16, 128


# ------------------------------------------------------- exact rounding --

def _round_binary(x: Fraction, mant: int, emin: int, emax: int) -> float:
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ex = max(e, emin)
    n = round(a / Fraction(2) ** (ex - mant))  # Fraction rounds half to even
    if n == 2 ** (mant + 1):
        n, ex = 2 ** mant, ex + 1
    if ex > emax:
        return sign * math.inf
    return sign * float(Fraction(n) * Fraction(2) ** (ex - mant))


def rn32(x) -> float:
    return _round_binary(Fraction(x), 23, -126, 127)


def rn16(x) -> float:
    return _round_binary(Fraction(x), 10, -14, 15)


def rnbf16(x) -> float:
    return _round_binary(Fraction(x), 7, -126, 127)


def f32_fma(a, b, c) -> float:
    return rn32(Fraction(a) * Fraction(b) + Fraction(c))


def f32_mul(a, b) -> float:
    return rn32(Fraction(a) * Fraction(b))


def f32_div(a, b) -> float:
    return rn32(Fraction(a) / Fraction(b))


def f32_sub(a, b) -> float:
    return rn32(Fraction(a) - Fraction(b))


def rint_even(x: float) -> int:
    return int(round(x))  # Python rounds half to even


def exp2_coeffs_exact() -> list[float]:
    """fp32 RNE of ln2^k / k!, k = 0..7, from a 60-digit ln 2."""
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    out = []
    for k in range(8):
        v = ln2 ** k / Decimal(math.factorial(k))
        out.append(rn32(Fraction(v)))
    return out


_C = None


def exp2s(y: float) -> float:
    global _C
    if _C is None:
        _C = exp2_coeffs_exact()
    if not (y >= -125.0):
        return 0.0
    n = rint_even(y)
    f = y - n  # exact for binary32 y
    p = _C[7]
    for k in range(6, -1, -1):
        p = f32_fma(p, f, _C[k])
    return float(Fraction(p) * Fraction(2) ** n)


# ------------------------------------------------------------ quantizers --

def quant_int4_exact(x):
    """Group-affine INT4 of one vector of binary32 values by exact rational
    steps: delta = rn16(rn32((max - min) / 15)) from the FP32 difference,
    m = rn16(min), code = clamp(rint_even(rn32(rn32(x - m) / delta)), 0, 15),
    all zero when delta is 0.  Returns (codes, delta, m) as Python values."""
    xs = [float(v) for v in x]
    mn, mx = min(xs), max(xs)
    d = rn16(Fraction(f32_div(f32_sub(mx, mn), 15.0)))
    m = rn16(Fraction(mn))
    if d == 0.0:
        return [0] * len(xs), d, m
    return [min(15, max(0, rint_even(f32_div(f32_sub(v, m), d)))) for v in xs], d, m


def quant_int8_exact(x):
    """Symmetric INT8 of one vector: s = rn16(rn32(max|x| / 127)),
    code = clamp(rint_even(rn32(x / s)), -127, 127), all zero when s is 0."""
    xs = [float(v) for v in x]
    s = rn16(Fraction(f32_div(max(abs(v) for v in xs), 127.0)))
    if s == 0.0:
        return [0] * len(xs), s
    return [min(127, max(-127, rint_even(f32_div(v, s)))) for v in xs], s


# --------------------------------------------------------------- rotation --

def sylvester(n: int) -> np.ndarray:
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32_recursive(x: np.ndarray) -> np.ndarray:
    """H_n x by the recursion H_2n x = [H_n a + H_n b, H_n a - H_n b] with
    FP32 adds; the outermost split is the stride-64 butterfly, applied last."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    if n == 1:
        return x.copy()
    a = fwht_f32_recursive(x[..., : n // 2])
    b = fwht_f32_recursive(x[..., n // 2:])
    return np.concatenate([a + b, a - b], axis=-1).astype(np.float32)


def inv_sqrt128_f32() -> np.float32:
    """fp32 RNE of 2^-3.5 from a 60-digit square root."""
    getcontext().prec = 60
    return np.float32(rn32(Fraction(Decimal(1) / (Decimal(8) * Decimal(2).sqrt()))))


# -------------------------------------------------------------- unpacking --

def _f16(lo: int, hi: int) -> float:
    return float(np.array([lo | (hi << 8)], np.uint16).view(np.float16)[0])


def unpack_block(block: np.ndarray):
    """block: uint8[2176] -> (kc[16][128], vc[16][128], kd[16], km[16], vd[16], vm[16])."""
    kc = np.zeros((PAGE, HD), np.int64)
    vc = np.zeros((PAGE, HD), np.int64)
    for t in range(PAGE):
        for ch in range(HD):
            byte = int(block[64 * t + ch // 2])
            kc[t, ch] = (byte >> (4 * (ch % 2))) & 15
    for ch in range(HD):
        for t in range(PAGE):
            byte = int(block[1024 + 8 * ch + t // 2])
            vc[t, ch] = (byte >> (4 * (t % 2))) & 15
    meta = []
    for base in (2048, 2112):
        d = [_f16(int(block[base + 4 * t]), int(block[base + 4 * t + 1])) for t in range(PAGE)]
        m = [_f16(int(block[base + 4 * t + 2]), int(block[base + 4 * t + 3])) for t in range(PAGE)]
        meta += [d, m]
    return kc, vc, *meta


# ----------------------------------------------------------------- decode --

def query_codes(q_bf16_bits: np.ndarray):
    """Rotated, symmetric INT8 query codes by explicit FP32 steps."""
    q = (q_bf16_bits.astype(np.uint32) << 16).view(np.float32)
    r = (fwht_f32_recursive(q) * inv_sqrt128_f32()).astype(np.float32)
    a = float(np.max(np.abs(r)))
    s = f32_div(a, 127.0)
    if s == 0.0:
        return np.zeros(HD, np.int64), 0.0, 0
    codes = np.array([min(127, max(-127, rint_even(f32_div(float(x), s)))) for x in r], np.int64)
    return codes, s, int(codes.sum())


def decode_one(pages, side_codes, side_scales, Hkv, q_bits, L, slot, g, table_row, scale_log2,
               pv_exact=False, sink=SINK, window=WINDOW, E=None):
    """One (query, q-head) attending [0, L): returns out[128] (f64), lse, and
    dicts of the integer intermediates keyed by position / logical page.
    sink / window: the protection budget s, w; E: the end of the cache (the
    recent window is [E - w, E)), L for a decode step."""
    E = L if E is None else E
    qc, s_q, S_q = query_codes(q_bits)
    c_q = f32_mul(s_q, scale_log2)
    qk, pcode, pv = {}, {}, {}
    parts = []
    # protected region: sinks and recent window
    prot = list(range(0, min(sink, L))) + list(range(max(sink, E - window), L))
    zs, rows = [], []
    for p in prot:
        row = p if p < sink else sink + p % window
        k8 = side_codes[slot, g, row, 0].astype(np.int64)
        d8 = int(np.dot(qc, k8))
        qk[p] = d8
        sk = float(np.array([side_scales[slot, g, row, 0]], np.uint16).view(np.float16)[0])
        zs.append(f32_mul(f32_mul(float(d8), sk), c_q))
        rows.append(row)
    zmax = max(zs) if zs else -math.inf
    A = np.zeros(HD)
    ell = 0.0
    for z, row in zip(zs, rows):
        e = exp2s(f32_sub(z, zmax))
        sv = float(np.array([side_scales[slot, g, row, 1]], np.uint16).view(np.float16)[0])
        v8 = side_codes[slot, g, row, 1].astype(np.int64)
        vhat = np.array([rnbf16(f32_mul(sv, float(c))) for c in v8])
        A += e * vhat
        ell += e
    if prot:
        parts.append((A, zmax, ell))
    # main region, one tile per logical page
    main_end = min(L, E - window)
    j = sink // PAGE
    while PAGE * j < main_end:
        kc, vc, kd, km, vd, vm = unpack_block(pages[table_row[j], g])
        n = min(PAGE, main_end - PAGE * j)
        z = []
        for t in range(n):
            D = int(np.dot(qc, kc[t]))
            qk[PAGE * j + t] = D
            z.append(f32_mul(f32_fma(kd[t], float(D), f32_mul(km[t], float(S_q))), c_q))
        zt = max(z)
        e = [exp2s(f32_sub(zz, zt)) for zz in z]
        u = [f32_mul(e[t], vd[t]) for t in range(n)]
        umax = max(u)
        ell = sum(e)
        mu = sum(e[t] * vm[t] for t in range(n))
        if pv_exact:
            A = np.array([sum(e[t] * (vd[t] * vc[t, ch] + vm[t]) for t in range(n))
                          for ch in range(HD)])
        else:
            if umax == 0.0:
                uc = [0] * n
            else:
                inv = f32_div(127.0, umax)
                uc = [min(127, max(0, rint_even(f32_mul(ut, inv)))) for ut in u]
            acc = np.array([sum(uc[t] * int(vc[t, ch]) for t in range(n)) for ch in range(HD)])
            for t in range(n):
                pcode[PAGE * j + t] = uc[t]
            pv[j] = acc
            A = (umax / 127.0) * acc.astype(np.float64) + mu
        parts.append((A, zt, ell))
        j += 1
    Z = max(p[1] for p in parts)
    num = sum(2.0 ** (p[1] - Z) * p[0] for p in parts)
    den = sum(2.0 ** (p[1] - Z) * p[2] for p in parts)
    return num / den, math.log(2) * (Z + math.log2(den)), qk, pcode, pv


def unpack_kv8_block(block: np.ndarray):
    """Independent reading of one KV8 block (4160 bytes): K codes [16][128]
    token-major, V codes [128][16] channel-major, then 16 FP16 key scales and
    16 FP16 value scales.  Returns (kc [16][128], vc [16][128], sk [16], sv [16])."""
    b = np.asarray(block, np.uint8)
    kc = b[:2048].view(np.int8).reshape(PAGE, HD).astype(np.int64)
    vc = b[2048:4096].view(np.int8).reshape(HD, PAGE).T.astype(np.int64)
    sk = [_f16(int(b[4096 + 2 * t]), int(b[4097 + 2 * t])) for t in range(PAGE)]
    sv = [_f16(int(b[4128 + 2 * t]), int(b[4129 + 2 * t])) for t in range(PAGE)]
    return kc, vc, sk, sv


def kv8_decode_one(pages, q_bits, L, g, table_row, scale_log2):
    """KV8 everywhere, one (sequence, q-head): every position through the
    protected path's rules.  Returns out[128] (f64), lse, {position: D8}."""
    qc, s_q, _ = query_codes(q_bits)
    c_q = f32_mul(s_q, scale_log2)
    zs, vrows, qk = [], [], {}
    for p in range(L):
        kc, vc, sk, sv = unpack_kv8_block(pages[table_row[p // PAGE], g])
        t = p % PAGE
        d8 = int(np.dot(qc, kc[t]))
        qk[p] = d8
        zs.append(f32_mul(f32_mul(float(d8), sk[t]), c_q))
        vrows.append(np.array([rnbf16(f32_mul(sv[t], float(c))) for c in vc[t]]))
    zmax = max(zs)
    A = np.zeros(HD)
    ell = 0.0
    for z, vh in zip(zs, vrows):
        e = exp2s(f32_sub(z, zmax))
        A += e * vh
        ell += e
    return A / ell, math.log(2) * (zmax + math.log2(ell)), qk



# ------------------------------------------------------- MXFP4 variant --

E2M1_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]  # magnitudes of codes 0..7


def mx_quant_block(x):
    """OCP MXFP4 block by exact rationals: E = floor(log2 amax) - 2 (clamped to
    [-127, 127]; -127 for an all-zero block), code = the grid magnitude nearest
    to |x| / 2^E (ties to the even code), saturated at 6, sign from x.
    Returns (codes [32], E8M0 byte)."""
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        E = -127
    else:
        E = 0
        while Fraction(2) ** (E + 1) <= amax:
            E += 1
        while Fraction(2) ** E > amax:
            E -= 1
        E = max(-127, min(127, E - 2))
    codes = []
    for v, f in zip(xs, x):
        y = abs(v) / Fraction(2) ** E
        best = min(range(8), key=lambda c: (abs(E2M1_GRID[c] - y), c % 2))
        if y > 6:
            best = 7
        codes.append(best | (8 if math.copysign(1.0, float(f)) < 0 else 0))
    return codes, E + 127


def e2m1(code) -> float:
    return float((-1 if code & 8 else 1) * E2M1_GRID[code & 7])


def unpack_mx_block(block: np.ndarray):
    """Independent reading of one MXFP4 block: (k [16][128], v [16][128]) dequantized exactly."""
    b = np.asarray(block, np.uint8)
    k = np.zeros((PAGE, HD))
    v = np.zeros((PAGE, HD))
    for t in range(PAGE):
        for j in range(HD):
            kc = (int(b[64 * t + j // 2]) >> (4 * (j % 2))) & 15
            vc = (int(b[1024 + 8 * j + t // 2]) >> (4 * (t % 2))) & 15
            k[t, j] = e2m1(kc) * 2.0 ** (int(b[2048 + 4 * t + j // 32]) - 127)
            v[t, j] = e2m1(vc) * 2.0 ** (int(b[2112 + 4 * t + j // 32]) - 127)
    return k, v


def mx_decode_one(pages, side_codes, side_scales, q_bits, L, slot, g, table_row, scale_log2,
                  sink=SINK, window=WINDOW):
    """MXFP4 variant, one (sequence, q-head): protected region as decode_one,
    main region [s, L-w) with z = fp32(bf16(q_rot) . k^) * c, FP32 exp2s weights
    relative to the region max, exact v^; exact merge."""
    qc, s_q, _ = query_codes(q_bits)
    c_q = f32_mul(s_q, scale_log2)
    q = (q_bits.astype(np.uint32) << 16).view(np.float32)
    r = (fwht_f32_recursive(q) * inv_sqrt128_f32()).astype(np.float32)
    qb = np.array([rnbf16(float(x)) for x in r])
    parts = []
    prot = list(range(0, min(sink, L))) + list(range(max(sink, L - window), L))
    zs, rows = [], []
    for p in prot:
        row = p if p < sink else sink + p % window
        d8 = int(np.dot(qc, side_codes[slot, g, row, 0].astype(np.int64)))
        sk = float(np.array([side_scales[slot, g, row, 0]], np.uint16).view(np.float16)[0])
        zs.append(f32_mul(f32_mul(float(d8), sk), c_q))
        rows.append(row)
    if zs:
        zmax = max(zs)
        A, ell = np.zeros(HD), 0.0
        for z, row in zip(zs, rows):
            e = exp2s(f32_sub(z, zmax))
            sv = float(np.array([side_scales[slot, g, row, 1]], np.uint16).view(np.float16)[0])
            A += e * np.array([rnbf16(f32_mul(sv, float(c))) for c in side_codes[slot, g, row, 1]])
            ell += e
        parts.append((A, zmax, ell))
    mz, mv = [], []
    for p in range(sink, max(sink, L - window)):
        kk, vv = unpack_mx_block(pages[table_row[p // PAGE], g])
        d = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qb, kk[p % PAGE]))
        mz.append(f32_mul(rn32(d), scale_log2))
        mv.append(vv[p % PAGE])
    if mz:
        zmax = max(mz)
        A, ell = np.zeros(HD), 0.0
        for z, vv in zip(mz, mv):
            e = exp2s(f32_sub(z, zmax))
            A += e * vv
            ell += e
        parts.append((A, zmax, ell))
    Z = max(p[1] for p in parts)
    num = sum(2.0 ** (p[1] - Z) * p[0] for p in parts)
    den = sum(2.0 ** (p[1] - Z) * p[2] for p in parts)
    return num / den, math.log(2) * (Z + math.log2(den))
