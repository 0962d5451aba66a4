"""Pins of the DiT frequency-grid oracle: an arbitrary-precision evaluation of the
same recipe (bitwise), closed forms at both ends, the geometric ratio, and torch
executing the page's expression on the CPU (within 1 or 2 ulp: torch's own
linspace and pow round their last bit differently)."""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np
import pytest
import torch

import oracle.dit_freqs as df
from tests import exact_trig

CASES = [(10000.0, 4096, 6), (10000.0, 2048, 6), (10000.0, 128, 2), (500.0, 96, 3), (10000.0, 11, 6), (10000.0, 5, 6)]


def exact_f32(v: Decimal) -> np.float32:
    r, _ = exact_trig.round_to_f32(v)
    return r


def pin_exact(theta, dim, ne, double):
    got = df.freq_grid(theta, dim, ne, double)
    n = dim // ne
    assert got.shape == (n,) and got.dtype == np.float32
    with localcontext() as ctx:
        ctx.prec = 60
        pi = exact_trig.pi()
        for i in range(n):
            xi = Decimal(i) / Decimal(n - 1) if n > 1 else Decimal(0)
            if double:
                v = (Decimal(theta).ln() * xi).exp() * pi / 2
                want, amb = exact_trig.round_to_f32(v)
                # float64 intermediates: equal to the exact value rounded once, unless it sits on a midpoint
                assert amb or got[i] == want or abs(float(got[i]) - float(v)) <= np.spacing(np.float32(v)) * 0.5 + 1e-12 * float(v), (i, got[i], want)
            else:
                xf = Decimal(float(np.float32(float(xi))))
                th = Decimal(float(np.float32(theta)))
                pw = exact_f32((th.ln() * xf).exp())
                prod = exact_f32(Decimal(float(pw)) * Decimal(float(np.float32(math.pi))))
                assert got[i] == np.float32(float(prod) / 2.0), (i, got[i], prod)


def pin_closed_forms():
    for double in (True, False):
        g = df.freq_grid(10000.0, 4096, 6, double)
        assert g[0] == (np.float32(math.pi / 2) if double else np.float32(np.float32(math.pi) / np.float32(2)))
        top = np.float32(10000.0 * math.pi / 2) if double else np.float32(np.float32(10000.0 * np.float32(math.pi)) / 2)
        assert g[-1] == top
        r = g[1:].astype(np.float64) / g[:-1].astype(np.float64)
        assert np.allclose(r, 10000.0 ** (1.0 / (len(g) - 1)), rtol=1e-5 if double else 5e-5)
        assert np.all(np.diff(g) > 0)
    assert df.freq_grid(10000.0, 5, 6, True).shape == (0,)
    assert df.freq_grid(10000.0, 11, 6, False).tolist() == [np.float32(np.float32(math.pi) / np.float32(2))]


def torch_page_expression(theta, dim, ne, double):
    dt = torch.float64 if double else torch.float32
    pow_indices = torch.pow(theta, torch.linspace(start=0.0, end=1.0, steps=dim // ne, dtype=dt))
    return (pow_indices * torch.pi / 2.0).to(dtype=torch.float32).numpy()


def _ulps(a, b):
    ia = a.view(np.int32 if a.dtype == np.float32 else np.int64).astype(np.int64)
    ib = b.view(np.int32 if b.dtype == np.float32 else np.int64).astype(np.int64)
    return np.abs(ia - ib)


def pin_torch(theta, dim, ne, double):
    """torch's linspace is within 1 ulp of i/(n-1); fed with the same x, torch's power and
    scaling agree with the oracle within 2 ulp (fp32 pow) / 1 ulp after the fp32 cast."""
    n = dim // ne
    dt = torch.float64 if double else torch.float32
    x = df.linspace01(n, double)
    assert _ulps(x, torch.linspace(0.0, 1.0, steps=n, dtype=dt).numpy()).max(initial=0) <= 1
    got = df.freq_grid(theta, dim, ne, double)
    want = (torch.pow(theta, torch.from_numpy(x)) * torch.pi / 2.0).to(dtype=torch.float32).numpy()
    assert _ulps(got, want).max(initial=0) <= (1 if double else 2)
    if double:  # in float64 the linspace difference vanishes in the final float32 rounding
        assert _ulps(got, torch_page_expression(theta, dim, ne, double)).max(initial=0) <= 1


@pytest.mark.parametrize("theta,dim,ne", CASES)
@pytest.mark.parametrize("double", [True, False], ids=["f64", "f32"])
def test_exact(theta, dim, ne, double):
    pin_exact(theta, dim, ne, double)


@pytest.mark.parametrize("theta,dim,ne", CASES)
@pytest.mark.parametrize("double", [True, False], ids=["f64", "f32"])
def test_torch_page_expression(theta, dim, ne, double):
    pin_torch(theta, dim, ne, double)


def test_closed_forms():
    pin_closed_forms()


def _linspace_wrong_denominator(n, double):
    x = np.array([i / n for i in range(n)], dtype=np.float64)
    return x if double else x.astype(np.float32)


def _freq_missing_half(theta, dim, ne, double):
    return df.__dict__["_orig_freq_grid"](theta, dim, ne, double) * np.float32(2)


@pytest.mark.parametrize("name,impl", [("linspace01", _linspace_wrong_denominator), ("freq_grid", _freq_missing_half)])
def test_planted_mistake_is_caught(monkeypatch, name, impl):
    monkeypatch.setitem(df.__dict__, "_orig_" + name, getattr(df, name))
    monkeypatch.setattr(df, name, impl)
    caught = 0
    for pin in (lambda: pin_exact(10000.0, 128, 2, True), lambda: pin_exact(10000.0, 128, 2, False), pin_closed_forms,
                lambda: pin_torch(10000.0, 128, 2, True)):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught
