"""Hand-made cache contents for degenerate cases of the main-region P-operand
rule: raw page bytes written directly (no quantizer runs), with every value
exactly representable, so that the expected codes and outputs follow by hand.
Inputs only; shared by the oracle's pins and the GPU parity tests.

A page here has every K code 0 and delta_k = 0, so a logit is
m_k * S_q * c_q; with the unit query below (all codes 127, S_q = 16256) one
unit of m_k is about 1.443 in base-2 units (scale 1/sqrt(128)).  Position 0
has (m_k, delta_v, m_v) = (mk0, dv0, mv0), the other 15 positions
(mk1, dv1, mv1); every V code is `code`."""
from __future__ import annotations

import numpy as np

BLOCK, OFF_VCODE, OFF_KMETA, OFF_VMETA = 2176, 1024, 2048, 2112

# name: (mk0, mk1, dv0, dv1, mv0, mv1, code)
CASES = {
    # the other weights near 2^-115 (normal FP32) and delta_v = 2^-24 (the
    # smallest FP16 subnormal), position 0 with delta_v = 0: u = e * delta_v
    # is 0 at position 0 and FP32-subnormal elsewhere, 127 / u_max overflows
    "u_max_subnormal": (100.0, 20.0, 0.0, 2.0 ** -24, 1.5, -0.5, 5),
    # the others 144 below position 0: exp2s returns 0 below -125
    "weights_cut_off": (100.0, 0.0, 1.0, 1.0, 1.5, -0.5, 5),
    # constant V vectors everywhere (delta_v = 0): u_max = 0, every code 0
    "u_max_zero": (100.0, 99.0, 0.0, 0.0, 1.5, -0.5, 5),
}


def _meta(blk, off, t, d, m):
    blk[off + 4 * t: off + 4 * t + 4] = np.array([d, m], np.float16).view(np.uint8)


def page(name: str) -> np.ndarray:
    """The page block (16 positions of one kv-head) of case `name`."""
    mk0, mk1, dv0, dv1, mv0, mv1, code = CASES[name]
    blk = np.zeros(BLOCK, np.uint8)
    blk[OFF_VCODE:OFF_KMETA] = code | (code << 4)
    for t in range(16):
        _meta(blk, OFF_KMETA, t, 0.0, mk0 if t == 0 else mk1)
        _meta(blk, OFF_VMETA, t, dv0 if t == 0 else dv1, mv0 if t == 0 else mv1)
    return blk


def unit_query(T: int, Hq: int) -> np.ndarray:
    """BF16 queries [T][Hq][128] with 1.0 in channel 0: rotated, every channel
    is 2^-3.5, so every INT8 code is 127 and S_q = 127 * 128."""
    q = np.zeros((T, Hq, 128), np.uint16)
    q[..., 0] = 0x3F80
    return q
