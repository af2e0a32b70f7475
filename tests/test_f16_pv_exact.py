"""Host check of the arithmetic behind the re-prefill attention's PV product on
the f16 MFMA: a V code byte masked in place gives f16 subnormals (low nibble c
-> c 2^-24, high nibble left in bits 4..7 -> 16 c 2^-24), P codes enter as f16
integers (16 uc against low nibbles, uc against high ones), and every product
and partial sum of a 16-position tile is then an integer multiple of 2^-24
small enough for FP32, so the sum is the integer PV times 2^-20 in any order.
The MFMA's own handling of subnormal f16 inputs is checked on the GPU by the
bit-exact int32 PV of the parity tests; this pins the encoding and the bound."""
import numpy as np


def _half(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_nibbles_masked_in_place_are_exact_subnormals():
    byte = np.arange(256, dtype=np.uint16)
    lo, hi = byte & 0x0F, (byte >> 4) & 0x0F
    assert np.array_equal(_half(byte & 0x000F), lo * 2.0 ** -24)
    assert np.array_equal(_half(byte & 0x00F0), 16 * hi * 2.0 ** -24)


def test_p_codes_are_exact_f16_integers():
    uc = np.arange(128, dtype=np.float32)
    for scale in (1, 16):
        assert np.array_equal(np.float16(uc * scale).astype(np.float32), uc * scale)


def test_tile_sums_are_exact_in_fp32_in_any_order():
    rng = np.random.default_rng(7)
    cases = [np.full(16, 127), rng.integers(0, 128, 16)] + [rng.integers(0, 128, 16) for _ in range(500)]
    vcases = [np.full(16, 15), rng.integers(0, 16, 16)] + [rng.integers(0, 16, 16) for _ in range(500)]
    for uc, c in zip(cases, vcases):
        exact = int((uc * c).sum())
        assert exact <= 16 * 127 * 15 < 2 ** 24 // 16
        # slots alternate low (scale 1 on V, 16 on P) and high (16 on V, 1 on P) nibbles
        terms = []
        for k in range(16):
            if k % 2 == 0:
                terms.append(np.float32(16 * uc[k]) * np.float32(c[k] * 2.0 ** -24))
            else:
                terms.append(np.float32(uc[k]) * np.float32(16 * c[k] * 2.0 ** -24))
        for order in (range(16), reversed(range(16)), rng.permutation(16)):
            acc = np.float32(0.0)
            for k in order:
                acc = np.float32(acc + terms[k])
            assert float(acc) == exact * 2.0 ** -20
        # the tile scale takes the 2^20 back exactly
        assert float(np.float32(acc) * np.float32(2.0 ** 20)) == exact
