"""Pins of the DiT frequency-grid oracle against what the page and the mathematics fix.

* linspace: bit for bit against torch.linspace on the CPU (the call the page prints),
  both dtypes, many lengths and a few other (start, end) pairs.
* the power: closed forms where the correctly rounded result is an IEEE basic operation
  (x = 0, 1, 2, -1 and 1/2: 1, theta, theta*theta, 1/theta, sqrt(theta)), and the platform
  libm within 1 ulp (equal almost always).
* the whole grid: torch evaluating the page's expression on the CPU -- 0 ulp for the
  float64 recipe, at most 2 ulp for the float32 one, where torch's own float32 pow may
  land one unit away from the correctly rounded power;
  closed forms at both ends and the geometric ratio.
* planted mistakes that these pins must catch.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.dit_freqs as df

CASES = [(10000.0, 4096, 6), (10000.0, 2048, 6), (10000.0, 128, 2), (500.0, 96, 3), (1.0e6, 256, 2),
         (2.5, 64, 1), (10000.0, 11, 6), (10000.0, 5, 6)]
LENGTHS = [0, 1, 2, 3, 4, 5, 7, 8, 17, 31, 32, 63, 64, 100, 341, 682, 1000, 1023, 4097]


def _uint(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint64 if x.dtype == np.float64 else np.uint32)


def _ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.view(np.int64 if a.dtype == np.float64 else np.int32).astype(np.int64)
    ib = b.view(np.int64 if b.dtype == np.float64 else np.int32).astype(np.int64)
    return np.abs(ia - ib)


def torch_page_expression(theta, dim, ne, double):
    dt = torch.float64 if double else torch.float32
    pow_indices = torch.pow(theta, torch.linspace(start=0.0, end=1.0, steps=dim // ne, dtype=dt))
    return (pow_indices * torch.pi / 2.0).to(dtype=torch.float32).numpy()


# ---------------------------------------------------------------------------
# pins (each a plain function, so the planted-mistake test can run them)
# ---------------------------------------------------------------------------

def pin_round_to_ieee_casts():
    """The exact rounding helper against numpy's IEEE float64 -> float32 conversion on doubles (a
    correctly rounded cast): random values, exact float32 midpoints, and the overflow boundary."""
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000))
    f32 = rng.standard_normal(500).astype(np.float32)
    vals += [float(np.float64(v) + np.float64(np.spacing(v)) / 2) for v in f32]  # exact midpoints
    flt_max = float(np.finfo(np.float32).max)
    vals += [flt_max, 2.0 ** 128 - 2.0 ** 103, 2.0 ** 128 - 2.0 ** 102, -(2.0 ** 128 - 2.0 ** 103), 2.0 ** 128]
    with np.errstate(over="ignore"):
        for v in vals:
            got = df.round_to(Fraction(v), False)
            want = np.float32(v)
            assert got.view(np.uint32) == want.view(np.uint32), (v, got, want)
    assert df.round_to(Fraction(2) ** 1024, True) == np.inf
    assert df.round_to(Fraction(1, 3), True) == np.float64(1.0) / np.float64(3.0)


def pin_linspace_torch():
    for double in (True, False):
        dt = torch.float64 if double else torch.float32
        for n in LENGTHS:
            got = df.linspace01(n, double)
            want = torch.linspace(0.0, 1.0, steps=n, dtype=dt).numpy()
            assert got.dtype == want.dtype and got.shape == want.shape
            assert np.array_equal(_uint(got), _uint(want)), (n, double, int((_uint(got) != _uint(want)).sum()))
        for a, b, n in ((-3.0, 5.0, 11), (1.0, 0.0, 9), (0.25, 7.5, 130), (-1.0, 1.0, 1001)):
            got = df.linspace(a, b, n, double)
            want = torch.linspace(a, b, steps=n, dtype=dt).numpy()
            assert np.array_equal(_uint(got), _uint(want)), (a, b, n, double)


def pin_pow_closed_forms():
    rng = np.random.default_rng(7)
    bases = [10000.0, 500.0, 1.0e6, 2.5, 3.0, 0.37] + list(rng.uniform(1.0, 1.0e5, 40))
    for b64 in bases:
        for double in (True, False):
            b = np.float64(b64) if double else np.float32(b64)
            f = np.float64 if double else np.float32
            assert df.pow_rn(float(b), 0.0, double) == f(1.0)
            assert df.pow_rn(float(b), 1.0, double) == b
            assert df.pow_rn(float(b), 2.0, double) == f(b * b)      # one IEEE multiply
            assert df.pow_rn(float(b), -1.0, double) == f(f(1.0) / b)  # one IEEE division
            assert df.pow_rn(float(b), 0.5, double) == np.sqrt(b)    # IEEE square root, correctly rounded
    assert df.pow_rn(4.0, 0.5, True) == 2.0 and df.pow_rn(2.0, 10.0, False) == np.float32(1024.0)


def pin_pow_libm():
    """The platform's float64 pow (within about half an ulp) agrees within one ulp, and exactly on
    almost every input."""
    rng = np.random.default_rng(11)
    thetas = rng.uniform(1.5, 1.0e6, 300)
    xs = rng.uniform(0.0, 1.0, 300)
    got = np.array([df.pow_rn(float(t), float(x), True) for t, x in zip(thetas, xs)])
    want = np.array([math.pow(float(t), float(x)) for t, x in zip(thetas, xs)])
    u = _ulps(got, want)
    assert u.max() <= 1 and (u == 0).mean() >= 0.98, (u.max(), (u == 0).mean())
    th32 = thetas.astype(np.float32)
    x32 = xs.astype(np.float32)
    got32 = np.array([df.pow_rn(float(t), float(x), False) for t, x in zip(th32, x32)], np.float32)
    want32 = np.array([math.pow(float(t), float(x)) for t, x in zip(th32, x32)]).astype(np.float32)
    u32 = _ulps(got32, want32)
    assert u32.max() <= 1 and (u32 == 0).mean() >= 0.98


def pin_grid_torch(theta, dim, ne, double):
    got = df.freq_grid(theta, dim, ne, double)
    want = torch_page_expression(theta, dim, ne, double)
    assert got.shape == want.shape and got.dtype == np.float32
    u = _ulps(got, want)
    assert u.max(initial=0) <= (0 if double else 2), (theta, dim, ne, double, u.max(initial=0))


def pin_grid_closed_forms():
    for double in (True, False):
        g = df.freq_grid(10000.0, 4096, 6, double)
        if double:
            assert g[0] == np.float32(math.pi / 2)
            assert g[-1] == np.float32((10000.0 * math.pi) / 2)
        else:
            assert g[0] == np.float32(np.float32(math.pi) / np.float32(2))
            assert g[-1] == np.float32(np.float32(np.float32(10000.0) * np.float32(math.pi)) / np.float32(2))
        r = g[1:].astype(np.float64) / g[:-1].astype(np.float64)
        assert np.allclose(r, 10000.0 ** (1.0 / (len(g) - 1)), rtol=1e-5 if double else 5e-5)
        assert np.all(np.diff(g) > 0)
    assert df.freq_grid(10000.0, 5, 6, True).shape == (0,)
    assert df.freq_grid(10000.0, 11, 6, False).tolist() == [np.float32(np.float32(math.pi) / np.float32(2))]
    assert df.freq_grid(1.0, 60, 6, True).tolist() == [np.float32(math.pi / 2)] * 10


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

def test_round_to_matches_ieee_casts():
    pin_round_to_ieee_casts()


def test_linspace_equals_torch_bitwise():
    pin_linspace_torch()


def test_pow_closed_forms():
    pin_pow_closed_forms()


def test_pow_against_libm():
    pin_pow_libm()


@pytest.mark.parametrize("theta,dim,ne", CASES)
@pytest.mark.parametrize("double", [True, False], ids=["f64", "f32"])
def test_grid_against_torch_page_expression(theta, dim, ne, double):
    pin_grid_torch(theta, dim, ne, double)


def test_grid_closed_forms():
    pin_grid_closed_forms()


def test_pow_refuses_undecidable_rounding():
    # a power that is exactly a rounding boundary cannot be decided from a 60-digit approximation:
    # b*b = 1 + 2**-11 + 2**-24 lies exactly halfway between two float32 values
    b = 1.0 + 2.0 ** -12
    with pytest.raises(ArithmeticError):
        df.pow_rn(b, 2.0, False)


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _linspace_correctly_rounded_ratio(start, end, n, double):
    dt = np.float64 if double else np.float32
    if n <= 0:
        return np.zeros(0, dt)
    if n == 1:
        return np.array([start], dt)
    return np.array([start + (end - start) * i / (n - 1) for i in range(n)], dtype=np.float64).astype(dt)


def _linspace_unfused_second_half(start, end, n, double):
    dt = np.float64 if double else np.float32
    if n <= 1:
        return np.array([start] * n, dt)
    s = dt(dt(dt(end) - dt(start)) / dt(n - 1))
    return np.array([dt(dt(start) + dt(s * dt(i))) if i < n // 2 else dt(dt(end) - dt(s * dt(n - 1 - i)))
                     for i in range(n)], dt)


def _pow_negated_exponent(base, x, double):
    return df.__dict__["_orig_pow_rn"](base, -x, double)


def _grid_missing_half(theta, dim, ne, double):
    return df.__dict__["_orig_freq_grid"](theta, dim, ne, double) * np.float32(2)


def _pow_truncated(base, x, double):
    r = df.__dict__["_orig_pow_rn"](base, x, double)
    return np.nextafter(r, np.float64(0) if double else np.float32(0)) if r * r != r else r


MISTAKES = [("linspace", _linspace_correctly_rounded_ratio), ("linspace", _linspace_unfused_second_half),
            ("pow_rn", _pow_negated_exponent), ("freq_grid", _grid_missing_half), ("pow_rn", _pow_truncated)]


@pytest.mark.parametrize("name,impl", MISTAKES, ids=[f"{n}-{f.__name__}" for n, f in MISTAKES])
def test_planted_mistake_is_caught(monkeypatch, name, impl):
    monkeypatch.setitem(df.__dict__, "_orig_" + name, getattr(df, name))
    monkeypatch.setattr(df, name, impl)
    pins = [pin_round_to_ieee_casts, pin_linspace_torch, pin_pow_closed_forms, pin_pow_libm, pin_grid_closed_forms,
            lambda: pin_grid_torch(10000.0, 4096, 6, True), lambda: pin_grid_torch(500.0, 96, 3, False)]
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ArithmeticError):
            caught += 1
    assert caught, f"no pin caught the planted mistake in {name}"
