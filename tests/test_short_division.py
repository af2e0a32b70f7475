"""The quantizer kernels divide by an FP16 step or scale d without a full
IEEE division: q0 = RN(a*y), r = RN(fma(-q0, d, a)), q = RN(fma(r, y, q0))
with y = RN(1/d).  Because d has at most 11 significant bits, the residual is
exact and q is the correctly rounded quotient RN(a/d), the division the
quantization rules (and the oracle) use, whenever a and a/d are normal
binary32 numbers.  With subnormal values q may differ in its last bits, but
such quotients are far below 1/2, so the code rint(q) never changes.  Checked
here on the host for every finite positive FP16 divisor against
exact-quotient neighbourhoods (including the smallest subnormal dividends)
and random dividends."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_short_divisor_quotient_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "short_division")
        subprocess.run(["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-mfma", "-o", exe,
                        os.path.join(HERE, "c", "short_division.c"), "-lm"], check=True)
        out = subprocess.run([exe, "600"], check=True, capture_output=True, text=True).stdout.split()
    bad, n, bad_normal, bad_code = (int(x) for x in out)
    assert n > 30_000 * 600
    assert bad_normal == 0, f"{bad_normal} normal-range quotients differ from RN(a/d)"
    assert bad_code == 0, f"{bad_code} quotients round to a different integer"
    assert bad < n // 10_000  # only the subnormal corner differs at all
