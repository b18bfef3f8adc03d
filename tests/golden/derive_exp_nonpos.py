"""Derivation of the polynomial inside the library's fp64 exponential for
non-positive arguments (exp_nonpos in the device helpers).

e^x = 2^n e^r with x = n ln 2 + r, |r| <= ln2 / 2 < 0.347 (Cody and Waite's
additive reduction), and e^r = 1 + r q(r) where q is the degree-8 polynomial
that interpolates f(r) = (e^r - 1) / r at the 9 Chebyshev points of the
first kind on [-0.347, 0.347]:

    r_k = 0.347 cos((2k + 1) pi / 18),  k = 0 .. 8   (r_4 = 0, f(0) = 1).

Everything is exact or carried at 80 significant digits: the node values by
`decimal` (exp, and cos from its Taylor series, pi to 110 digits), the
Vandermonde system solved in rational arithmetic (`fractions`), and each
monomial coefficient rounded once to the nearest double.

    python tests/golden/derive_exp_nonpos.py    # prints the 9 coefficients
"""
from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 80

PI = Decimal("3.14159265358979323846264338327950288419716939937510582097494459230781640628"
             "620899862803482534211706798214808651")
HALF_WIDTH = Decimal("0.347")
DEGREE = 8


def _cos(x):
    x = Decimal(x)
    s, t, k = Decimal(0), Decimal(1), 0
    while abs(t) > Decimal(10) ** -78:
        s += t
        t = -t * x * x / ((2 * k + 1) * (2 * k + 2))
        k += 1
    return s


def _f(r):
    """(e^r - 1) / r, with its limit 1 at r = 0."""
    if r == 0:
        return Decimal(1)
    return (r.exp() - 1) / r


def nodes():
    n = DEGREE + 1
    mid = n // 2
    return [Decimal(0) if k == mid else HALF_WIDTH * _cos((2 * k + 1) * PI / (2 * n))
            for k in range(n)]


def coefficients():
    """Monomial coefficients c_0 .. c_8 of the interpolant, as Fractions."""
    xs = [Fraction(r) for r in nodes()]
    ys = [Fraction(_f(r)) for r in nodes()]
    n = len(xs)
    A = [[x ** j for j in range(n)] + [y] for x, y in zip(xs, ys)]
    for c in range(n):
        p = max(range(c, n), key=lambda i: abs(A[i][c]))
        A[c], A[p] = A[p], A[c]
        for i in range(n):
            if i != c and A[i][c] != 0:
                m = A[i][c] / A[c][c]
                A[i] = [u - m * v for u, v in zip(A[i], A[c])]
    return [A[i][n] / A[i][i] for i in range(n)]


def double_coefficients():
    """The coefficients rounded once to binary64."""
    return [float(c) for c in coefficients()]


if __name__ == "__main__":
    for j, c in enumerate(double_coefficients()):
        print(f"c{j} = {c.hex()}")
