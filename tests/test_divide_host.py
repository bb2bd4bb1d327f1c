"""The quantize kernels divide w / scale as RN(q + r y) with y = RN(1 / scale), q = RN(w y) and
r = w - scale q exact (csrc/divide.h), and claim the IEEE quotient. CPU checks of that claim:
  * the header itself, compiled for the host, against IEEE division on 1.2e8 random and 9e7
    adversarial operand pairs (tests/host/check_divide.cpp);
  * the same three steps in exact rational arithmetic over every pair of significands of binary
    formats with 4 to 9 significand bits (dividends over two binades), every rounding to nearest even.
The grid decision rint(w / scale) is taken on this quotient ([guide] "The code, line by line"), so an
exact tie or a near-half value rounds as the oracle's IEEE division does."""
import math
import os
import shutil
import subprocess
from fractions import Fraction

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_divide_header_matches_ieee_division(tmp_path):
    exe = tmp_path / "check_divide"
    src = os.path.join(HERE, "host", "check_divide.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), src], check=True)
    r = subprocess.run([str(exe), "120000000", "30000000", "7"], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0 and "mismatches=0" in r.stdout, r.stdout


def _rn(x: Fraction, p: int) -> Fraction:
    """x rounded to p significant bits, ties to even (no exponent range limits)."""
    if x == 0:
        return Fraction(0)
    s, x = (-1, -x) if x < 0 else (1, x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    m = x / Fraction(2) ** (e - p + 1)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    return s * fl * Fraction(2) ** (e - p + 1)


@pytest.mark.parametrize("p", [4, 5, 6, 7, 8, 9])
def test_three_step_quotient_exhaustive_in_narrow_formats(p):
    sigs = [Fraction(2 ** (p - 1) + k, 2 ** (p - 1)) for k in range(2 ** (p - 1))]
    bad = 0
    for b in sigs:
        y = _rn(1 / b, p)
        for a0 in sigs:
            for a in (a0, a0 / 2):
                q = _rn(a * y, p)
                r = _rn(a - b * q, p)  # the fused multiply-add's one rounding (exact whenever representable)
                bad += _rn(q + r * y, p) != _rn(a / b, p)
    assert bad == 0
    assert math.isfinite(float(sigs[-1]))
