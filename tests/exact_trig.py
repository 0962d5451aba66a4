"""Arbitrary-precision reference values for the rotary tables (test helper).

Independent of the oracle and of libm: pi from Machin's formula, the inverse
frequency base**(-2i/d) as exp(-(2i/d) ln base) with Python's decimal module,
cos and sin from their Taylor series after reduction modulo 2*pi, and an
exact round-to-nearest-even of the result to fp32 decided by comparing exact
decimal distances to the neighbouring fp32 values.
"""
from __future__ import annotations

import functools
from decimal import Decimal, localcontext

import numpy as np

PREC = 60


def _atan_inv(n: int) -> Decimal:
    """atan(1/n) by its alternating series."""
    x = Decimal(1) / n
    x2 = x * x
    term = x
    total = Decimal(0)
    k = 0
    eps = Decimal(10) ** (-(PREC + 5))
    while abs(term) > eps:
        total += term / (2 * k + 1) if k % 2 == 0 else -term / (2 * k + 1)
        term *= x2
        k += 1
    return total


@functools.lru_cache(maxsize=None)
def pi() -> Decimal:
    with localcontext() as ctx:
        ctx.prec = PREC + 10
        return 16 * _atan_inv(5) - 4 * _atan_inv(239)


def cos_sin(theta: Decimal):
    """(cos theta, sin theta) to about PREC digits."""
    with localcontext() as ctx:
        ctx.prec = PREC + 10
        two_pi = 2 * pi()
        r = theta - two_pi * (theta / two_pi).to_integral_value(rounding="ROUND_FLOOR")
        r2 = r * r
        c = Decimal(0)
        s = Decimal(0)
        tc = Decimal(1)  # r^(2k) / (2k)!
        ts = r  # r^(2k+1) / (2k+1)!
        k = 0
        eps = Decimal(10) ** (-(PREC + 5))
        while abs(tc) > eps or abs(ts) > eps:
            sign = 1 if k % 2 == 0 else -1
            c += sign * tc
            s += sign * ts
            tc = tc * r2 / ((2 * k + 1) * (2 * k + 2))
            ts = ts * r2 / ((2 * k + 2) * (2 * k + 3))
            k += 1
        return +c, +s


def inv_freq(base: float, dim: int, i: int) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = PREC + 10
        return (-(Decimal(2 * i) / Decimal(dim)) * Decimal(base).ln()).exp()


def round_to_f32(v: Decimal):
    """(nearest fp32 by exact comparison, ambiguous) where ambiguous means v sits
    within 1e-20 of an fp32 spacing from the midpoint between two fp32 values."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    with localcontext() as ctx:
        ctx.prec = PREC + 10
        dists = sorted((abs(Decimal(float(c)) - v), i) for i, c in enumerate(cands))
        best = cands[dists[0][1]]
        spacing = abs(Decimal(float(cands[dists[1][1]])) - Decimal(float(best)))
        ambiguous = (dists[1][0] - dists[0][0]) <= spacing * Decimal("1e-20")
    return np.float32(best), ambiguous


def table_entry(base: float, dim: int, p: int, i: int):
    """Correctly rounded fp32 (cos, sin) of p * base**(-2i/dim), plus an ambiguity flag."""
    with localcontext() as ctx:
        ctx.prec = PREC + 10
        theta = Decimal(p) * inv_freq(base, dim, i)
        c, s = cos_sin(theta)
    cf, ca = round_to_f32(c)
    sf, sa = round_to_f32(s)
    return cf, sf, (ca or sa)


@functools.lru_cache(maxsize=None)
def exact_axis_tables(length: int, dim: int, base: float):
    cos = np.empty((length, dim // 2), np.float32)
    sin = np.empty((length, dim // 2), np.float32)
    amb = np.zeros((length, dim // 2), bool)
    for p in range(length):
        for i in range(dim // 2):
            cos[p, i], sin[p, i], amb[p, i] = table_entry(base, dim, p, i)
    return cos, sin, amb
