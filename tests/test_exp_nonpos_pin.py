"""The library's fp64 exponential for non-positive arguments (exp_nonpos,
used by every label-smoothed row sum and by the linear classifier's merge),
pinned on the CPU without a GPU:

1. its polynomial coefficients, read from the device source, are exactly
   the once-rounded coefficients of the 9-point Chebyshev interpolant that
   tests/golden/derive_exp_nonpos.py derives in exact arithmetic;
2. its operation sequence, replayed here with every fma rounded once (exact
   rational arithmetic, then one rounding to binary64), stays within
   4e-14 relative of e^x computed to 60 digits by `decimal`, over a dense
   grid of [-40, 0] and seeded random points, and gives e^0 = 1 exactly.

Replaying the sequence is what makes this a pin of the device code: a wrong
coefficient, a dropped term, a wrong reduction constant or a wrong use of
the integer n all fail (2)."""
import os
import random
import re
import struct
from decimal import Decimal, localcontext
from fractions import Fraction

import pytest

from tests.golden import derive_exp_nonpos as DER

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "vocab_softmax_cross_row_amd", "csrc", "ce_device.h")


def _function_text():
    text = open(SRC).read()
    i = text.index("double exp_nonpos(double x)")
    return text[i:text.index("\n}\n", i)]


def _hexfloat(tok):
    return float.fromhex(tok)


def _parse():
    body = _function_text()
    consts = {name: float(val) for name, val in
              re.findall(r"constexpr double (\w+) = ([0-9.eE+-]+);", body)}
    first = re.search(r"double q = (0x[0-9a-fp.+-]+);", body).group(1)
    rest = re.findall(r"q = fma\(q, r, ([0-9a-fx.p+-]+)\);", body)
    # Horner order: highest degree first
    coeffs = [_hexfloat(first)] + [_hexfloat(t) if t.startswith("0x") else float(t)
                                   for t in rest]
    return consts, coeffs[::-1]     # c0 .. c8


def _fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _int32_low_word(d):
    lo = struct.unpack("<Q", struct.pack("<d", d))[0] & 0xFFFFFFFF
    return lo - (1 << 32) if lo >= (1 << 31) else lo


def _exp_nonpos(x, consts, c):
    """The device function's steps, each fma rounded once."""
    x = -1000.0 if x < -1000.0 else x
    a = _fma(x, consts["kInvLn2"], consts["kShift"])
    n = a - consts["kShift"]
    r = _fma(n, -consts["kLn2"], x)
    q = c[8]
    for j in range(7, -1, -1):
        q = _fma(q, r, c[j])
    import math
    return math.ldexp(_fma(q, r, 1.0), _int32_low_word(a))


def test_coefficients_are_the_derived_interpolant():
    _, c = _parse()
    assert len(c) == 9
    assert c == DER.double_coefficients()
    assert c[0] == 1.0


def test_relative_error_against_60_digit_exp():
    consts, c = _parse()
    assert consts["kShift"] == 1.5 * 2.0 ** 52
    xs = [-40.0 * i / 12000 for i in range(12001)]
    rng = random.Random(20240611)
    xs += [-rng.uniform(0.0, 40.0) for _ in range(4000)]
    xs += [-0.5 * 0.6931471805599453 * k for k in range(1, 116)]   # reduction boundaries
    worst = 0.0
    with localcontext() as ctx:
        ctx.prec = 60
        for x in xs:
            got = _exp_nonpos(x, consts, c)
            ref = Decimal(x).exp()
            err = abs((Decimal(got) - ref) / ref)
            worst = max(worst, float(err))
    print(f"exp_nonpos: largest relative error {worst:.3e} over {len(xs)} points")
    assert worst <= 4e-14, f"largest relative error {worst:.3e}"
    assert _exp_nonpos(0.0, consts, c) == 1.0
    assert _exp_nonpos(-2000.0, consts, c) == 0.0


@pytest.mark.parametrize("bad", range(9))
def test_a_wrong_coefficient_is_caught(bad):
    """Negative control: one coefficient off by one part in 10^3 breaks the
    error bound, so the bound does see every coefficient, the last one
    (weight r^9 <= 7e-5) included."""
    consts, c = _parse()
    c = list(c)
    c[bad] *= 1.0 + 1e-3
    worst = 0.0
    with localcontext() as ctx:
        ctx.prec = 60
        for i in range(2001):
            x = -40.0 * i / 2000
            got = _exp_nonpos(x, consts, c)
            ref = Decimal(x).exp()
            worst = max(worst, float(abs((Decimal(got) - ref) / ref)))
    assert worst > 4e-14
