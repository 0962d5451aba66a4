"""Pins of the patchify oracle: the page's stated packing order on a 2x2 golden
example, an element-by-element brute force of the index formula, round trips
and planted mistakes."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle.patchify as pf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "patchify_2x2.txt")


def load_golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, *nums = line.split()
        vals[key] = np.array([float(n) for n in nums], np.float32)
    return vals


def pin_golden():
    g = load_golden()
    x = g["input"].reshape(1, 1, 1, 2, 2)
    np.testing.assert_array_equal(pf.patchify(x, 2).reshape(-1), g["output"])
    np.testing.assert_array_equal(pf.unpatchify(g["output"].reshape(1, 4, 1, 1, 1), 2), x)


def pin_brute_force(shape=(2, 3, 2, 6, 8), p=2, seed=1):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    y = pf.patchify(x, p)
    B, C, F, H, W = shape
    assert y.shape == (B, C * p * p, F, H // p, W // p)
    for b in range(B):
        for c in range(C):
            for f in range(F):
                for yy in range(H):
                    for xx in range(W):
                        hh, ph = divmod(yy, p)
                        ww, pw = divmod(xx, p)
                        assert y[b, (c * p + pw) * p + ph, f, hh, ww] == x[b, c, f, yy, xx]


def pin_round_trip(seed=2):
    rng = np.random.default_rng(seed)
    for shape, p in (((1, 3, 4, 8, 12), 4), ((2, 2, 1, 6, 6), 3), ((1, 5, 2, 16, 8), 8), ((1, 1, 1, 3, 5), 1)):
        x = rng.integers(0, 1 << 15, size=shape).astype(np.uint16)
        np.testing.assert_array_equal(pf.unpatchify(pf.patchify(x, p), p), x)
        y = rng.integers(0, 1 << 15, size=pf.patchify(x, p).shape).astype(np.uint16)
        np.testing.assert_array_equal(pf.patchify(pf.unpatchify(y, p), p), y)


ALL_PINS = [("golden", pin_golden), ("brute", pin_brute_force),
            ("brute_p3", lambda: pin_brute_force((1, 2, 1, 6, 9), 3, 3)), ("round_trip", pin_round_trip)]


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(name, pin):
    pin()


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        pf.patchify(np.zeros((1, 1, 1, 5, 4)), 2)
    with pytest.raises(ValueError):
        pf.unpatchify(np.zeros((1, 3, 1, 2, 2)), 2)


def _patchify_h_w_swapped(x, p):
    B, C, F, H, W = x.shape
    y = x.reshape(B, C, F, H // p, p, W // p, p).transpose(0, 1, 4, 6, 2, 3, 5)  # (c, h-offset, w-offset)
    return np.ascontiguousarray(y).reshape(B, C * p * p, F, H // p, W // p)


def _patchify_offsets_outermost(x, p):
    B, C, F, H, W = x.shape
    y = x.reshape(B, C, F, H // p, p, W // p, p).transpose(0, 6, 4, 1, 2, 3, 5)  # (w-off, h-off, c)
    return np.ascontiguousarray(y).reshape(B, C * p * p, F, H // p, W // p)


@pytest.mark.parametrize("impl", [_patchify_h_w_swapped, _patchify_offsets_outermost])
def test_planted_mistake_is_caught(monkeypatch, impl):
    monkeypatch.setattr(pf, "patchify", impl)
    caught = []
    for name, pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(name)
    assert caught


def _unpatchify_h_w_swapped(y, p):
    B, Cpp, F, Hp, Wp = y.shape
    C = Cpp // (p * p)
    x = y.reshape(B, C, p, p, F, Hp, Wp).transpose(0, 1, 4, 5, 2, 6, 3)  # reads (c, h-offset, w-offset)
    return np.ascontiguousarray(x).reshape(B, C, F, Hp * p, Wp * p)


def _unpatchify_frames_transposed(y, p):
    B, Cpp, F, Hp, Wp = y.shape
    C = Cpp // (p * p)
    x = y.reshape(B, C, p, p, F, Hp, Wp).transpose(0, 4, 1, 5, 3, 6, 2)  # frames and channels swapped
    return np.ascontiguousarray(x).reshape(B, C, F, Hp * p, Wp * p)


@pytest.mark.parametrize("impl", [_unpatchify_h_w_swapped, _unpatchify_frames_transposed])
def test_planted_mistake_in_the_inverse_is_caught(monkeypatch, impl):
    monkeypatch.setattr(pf, "unpatchify", impl)
    caught = []
    for name, pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(name)
    assert caught
