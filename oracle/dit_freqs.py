"""Plain CPU oracle for the LTX DiT RoPE frequency grid.

TEST INFRASTRUCTURE ONLY (like oracle.rope): only tests/, the graft entry
point's smoke() and bench.py's CPU leg import it; the library never does.

What it computes (sglang PR #24660 page, "Key source snippets", the LTX DiT's
RoPE frequency generation; "Implementation breakdown", step 2: the grid is
generated on the target device in the requested precision, float32 or
float64, keeping the official rounding trajectory):

    n      = dim // num_rope_elems
    x      = linspace(start=0, end=1, steps=n)   in the working dtype
    p      = theta ** x                           in the working dtype
    freqs  = (p * pi / 2).to(float32)

Readings (the page prints the calls, not their rounding), each step rounded
to the working dtype, round to nearest even:

* linspace is torch.linspace, the call the page prints: a rounded step
  s = (end - start) / (n - 1); the first n // 2 values are start + s*i and
  the others end - s*(n - 1 - i), each with the product exact and one
  rounding at the end (a fused multiply-add); n = 1 gives [start].
* theta ** x is the correctly rounded power in the working dtype; for
  float32, theta (a Python float) is first rounded to float32, as torch does
  with a scalar base and a float32 exponent.  The bits of a device's own pow
  routine are not printed anywhere, so bit identity with any particular pow
  implementation cannot be checked beyond that routine's error bound.
* p * pi uses pi rounded to the working dtype and is rounded once; the
  division by 2 is exact; the float64 recipe rounds once more to float32.

Every rounding is done here exactly: values are exact rationals (fractions)
or 60-digit decimals of the power, rounded once to the target format, and a
decimal power too close to a rounding boundary to be decided raises.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

_PREC = 60  # decimal digits of the power before its one rounding


def round_to(v: Fraction, double: bool):
    """v rounded to nearest, ties to even, in float64 (double) or float32.  Magnitudes from halfway
    between the largest finite value and the next power of two upward round to infinity (IEEE
    overflow under round to nearest)."""
    emax, mant = (1024, 53) if double else (128, 24)
    if abs(v) >= Fraction(2) ** emax - Fraction(2) ** (emax - mant - 1):
        inf = np.float64(np.inf) if double else np.float32(np.inf)
        return inf if v > 0 else -inf
    if double:
        return np.float64(v.numerator / v.denominator)  # Python's int division rounds correctly
    g = np.float32(v.numerator / v.denominator)  # within one float32 step of the answer
    cands = {float(g), float(np.nextafter(g, np.float32(-np.inf))), float(np.nextafter(g, np.float32(np.inf)))}
    best = None
    for c in sorted(cands):
        if math.isinf(c):
            continue
        d = abs(Fraction(c) - v)
        even = (int(np.array(c, np.float32).view(np.uint32)) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def linspace(start: float, end: float, steps: int, double: bool) -> np.ndarray:
    """torch.linspace(start, end, steps) in float64 (double) or float32, as read above."""
    dt = np.float64 if double else np.float32
    if steps <= 0:
        return np.zeros(0, dt)
    a = round_to(Fraction(start), double)
    b = round_to(Fraction(end), double)
    if steps == 1:
        return np.array([a], dt)
    s = Fraction(float(round_to((Fraction(float(b)) - Fraction(float(a))) / (steps - 1), double)))
    out = np.empty(steps, dt)
    for i in range(steps):
        if i < steps // 2:
            out[i] = round_to(Fraction(float(a)) + s * i, double)
        else:
            out[i] = round_to(Fraction(float(b)) - s * (steps - 1 - i), double)
    return out


def linspace01(n: int, double: bool) -> np.ndarray:
    return linspace(0.0, 1.0, n, double)


def pow_rn(base: float, x: float, double: bool):
    """base ** x correctly rounded to float64 (double) or float32; base and x are taken as the
    exact values of the given floats (already in the working dtype) and base > 0."""
    if x == 0.0:
        return round_to(Fraction(1), double)
    with localcontext() as ctx:
        ctx.prec = _PREC
        v = (Decimal(float(base)).ln() * Decimal(float(x))).exp()
    vf = Fraction(v)
    r = round_to(vf, double)
    # the decimal value is within 10**-(_PREC - 5) relative of the exact power; refuse to decide
    # when a rounding boundary (a midpoint between neighbours) lies closer than that
    nb = np.nextafter(r, np.inf if vf > Fraction(float(r)) else -np.inf)
    mid = (Fraction(float(r)) + Fraction(float(nb))) / 2
    if abs(vf - mid) <= vf * Fraction(1, 10 ** (_PREC - 5)):
        raise ArithmeticError(f"pow({base}, {x}) too close to a rounding boundary to decide")
    return r


def _halved_f32(prod) -> np.float32:
    """prod / 2 (exact) rounded to float32; an overflowed product stays infinite."""
    if math.isinf(float(prod)):
        return np.float32(prod)
    return round_to(Fraction(float(prod)) / 2, False)


def freq_grid(theta: float, dim: int, num_rope_elems: int, double_precision: bool) -> np.ndarray:
    """The float32 grid of dim // num_rope_elems frequencies, float64 or float32 recipe."""
    n = dim // num_rope_elems
    x = linspace01(n, double_precision)
    out = np.empty(n, np.float32)
    if double_precision:
        pi = Fraction(math.pi)
        for i, xi in enumerate(x):
            p = pow_rn(theta, float(xi), True)
            prod = round_to(Fraction(float(p)) * pi, True)
            out[i] = _halved_f32(prod)
        return out
    th = float(np.float32(theta))
    pi = Fraction(float(np.float32(math.pi)))
    for i, xi in enumerate(x):
        p = pow_rn(th, float(xi), False)
        prod = round_to(Fraction(float(p)) * pi, False)
        out[i] = _halved_f32(prod)
    return out
