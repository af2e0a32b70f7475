"""Hand-made cache contents for degenerate cases of the main-region P-operand
rule: raw page bytes written directly (no quantizer runs), with every value
chosen exactly representable, so the expected codes and outputs follow by
hand.  Inputs only; shared by the oracle's pins and the GPU parity tests."""
from __future__ import annotations

import numpy as np

BLOCK, OFF_VCODE, OFF_KMETA, OFF_VMETA = 2176, 1024, 2048, 2112
TINY_PAGE_Z_GAP_M = (100.0, 20.0)  # m_k of position 0 and of the others
TINY_PAGE_V = (1.5, -0.5, 5)       # m_v of position 0, of the others, and the V code


def _meta(blk, off, t, d, m):
    blk[off + 4 * t: off + 4 * t + 4] = np.array([d, m], np.float16).view(np.uint8)


def tiny_weight_page() -> np.ndarray:
    """One page block (16 positions of one kv-head).  K codes 0 with
    delta_k = 0, so a logit is m_k * S_q * c_q: m_k = 100 at position 0 and 20
    elsewhere, which for a query whose codes are all 127 puts the other 15
    positions about 115 below position 0 in base-2 units (weights near
    2^-115, normal FP32).  Every V code is 5; position 0 has delta_v = 0 and
    m_v = 1.5, the others delta_v = 2^-24 (the smallest FP16 subnormal) and
    m_v = -0.5.  Then u = e * delta_v is 0 at position 0 and FP32-subnormal
    elsewhere, and 127 / u_max overflows to infinity."""
    blk = np.zeros(BLOCK, np.uint8)
    blk[OFF_VCODE:OFF_KMETA] = 0x55  # code 5 in both nibbles of every byte
    m0, m1 = TINY_PAGE_Z_GAP_M
    v0, v1, _ = TINY_PAGE_V
    for t in range(16):
        _meta(blk, OFF_KMETA, t, 0.0, m0 if t == 0 else m1)
        _meta(blk, OFF_VMETA, t, 0.0 if t == 0 else 2.0 ** -24, v0 if t == 0 else v1)
    return blk


def unit_query(T: int, Hq: int) -> np.ndarray:
    """BF16 queries [T][Hq][128] with 1.0 in channel 0: rotated, every channel
    is 2^-3.5, so every INT8 code is 127 and S_q = 127 * 128."""
    q = np.zeros((T, Hq, 128), np.uint16)
    q[..., 0] = 0x3F80
    return q
