"""Exact / high-precision brute force used to pin the fp64 oracle.

Written independently of ``oracle/``: rational arithmetic (``fractions.Fraction``)
for everything that is a finite sum of products, and 40-digit ``decimal`` for
exp and sqrt. Pure-Python loops, meant for matrices of a few rows and columns.
"""
from __future__ import annotations

import decimal
from decimal import Decimal
from fractions import Fraction

CTX = decimal.Context(prec=40)


def F(x) -> Fraction:
    return Fraction(float(x))


def mat(x):
    """numpy 1-D/2-D array -> nested lists of Fractions."""
    if getattr(x, "ndim", 1) == 1:
        return [F(v) for v in x]
    return [[F(v) for v in row] for row in x]


def mm(A, B):
    """Exact product of nested-list Fraction matrices A[m][k], B[k][n]."""
    m, k, n = len(A), len(B), len(B[0])
    assert all(len(r) == k for r in A)
    return [[sum((A[i][p] * B[p][j] for p in range(k)), Fraction(0)) for j in range(n)]
            for i in range(m)]


def D(q) -> Decimal:
    if isinstance(q, Fraction):
        return CTX.divide(Decimal(q.numerator), Decimal(q.denominator))
    return CTX.create_decimal(q)


def dexp(x: Decimal) -> Decimal:
    return CTX.exp(x)


def dsqrt(x: Decimal) -> Decimal:
    return CTX.sqrt(x)


LN2 = CTX.ln(Decimal(2))


def softmax_row(xs):
    xs = [D(x) for x in xs]
    mx = max(xs)
    es = [dexp(CTX.subtract(x, mx)) for x in xs]
    s = sum(es, Decimal(0))
    return [CTX.divide(e, s) for e in es]


def layernorm_row(xs, eps, gamma=None, beta=None):
    """xs: Fractions. Mean and biased variance exactly, then the root in decimal."""
    n = len(xs)
    mu = sum(xs, Fraction(0)) / n
    var = sum(((x - mu) ** 2 for x in xs), Fraction(0)) / n
    r = dsqrt(D(var + F(eps)))
    out = []
    for j, x in enumerate(xs):
        y = CTX.divide(D(x - mu), r)
        if gamma is not None:
            y = CTX.multiply(y, D(gamma[j]))
        if beta is not None:
            y = CTX.add(y, D(beta[j]))
        out.append(y)
    return out


def rmsnorm_row(xs, eps, w=None):
    n = len(xs)
    ms = sum((x * x for x in xs), Fraction(0)) / n
    r = dsqrt(D(ms + F(eps)))
    out = []
    for j, x in enumerate(xs):
        y = CTX.divide(D(x), r)
        if w is not None:
            y = CTX.multiply(y, D(w[j]))
        out.append(y)
    return out


def round_bf16_exact(q: Fraction) -> Fraction:
    """Round a rational to the nearest bf16 value (8 significant bits, binary32
    exponent range, spacing 2**-133 below 2**-126), ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2**(e-1) <= a < 2**e
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e <= a:
        e += 1
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    step_exp = max(e - 8, -133)
    step = Fraction(2) ** step_exp
    t = a / step
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * step


def dec_to_frac(x: Decimal) -> Fraction:
    return Fraction(x)
