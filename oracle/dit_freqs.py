"""Plain CPU oracle for the LTX DiT RoPE frequency grid.

TEST INFRASTRUCTURE ONLY (like oracle.rope).

What it computes (sglang PR #24660 page, "Key source snippets", the LTX DiT's
RoPE frequency generation, and "Implementation breakdown", step 2: generated
directly in the chosen precision instead of a NumPy-cached grid):

    n      = dim // num_rope_elems
    x      = linspace(0, 1, n)        in the working dtype (float64 or float32)
    p      = theta ** x               in the working dtype
    freqs  = (p * pi / 2).to(float32)

Readings (the page prints the calls, not their rounding): linspace(0, 1, n)
holds i / (n - 1) correctly rounded to the working dtype (just 0 for n = 1,
nothing for n = 0); theta ** x is one power in the working dtype (for
float32, theta is first rounded to float32 and the power is the float32
rounding of the float64 power of the float32 operands); the product with pi
uses pi rounded to the working dtype and is rounded to it; the division by 2
is exact; the float64 path rounds once more to float32 at the end.
"""
from __future__ import annotations

import math

import numpy as np


def linspace01(n: int, double: bool) -> np.ndarray:
    if n <= 0:
        return np.zeros(0, np.float64 if double else np.float32)
    if n == 1:
        return np.zeros(1, np.float64 if double else np.float32)
    x = np.array([i / (n - 1) for i in range(n)], dtype=np.float64)  # correctly rounded division
    return x if double else x.astype(np.float32)  # exact rational -> float64 -> float32 (see module note)


def freq_grid(theta: float, dim: int, num_rope_elems: int, double_precision: bool) -> np.ndarray:
    n = dim // num_rope_elems
    x = linspace01(n, double_precision)
    if double_precision:
        p = np.array([math.pow(theta, float(v)) for v in x], dtype=np.float64)
        return (p * math.pi / 2.0).astype(np.float32)
    th = float(np.float32(theta))
    p = np.array([np.float32(math.pow(th, float(v))) for v in x], dtype=np.float32)
    prod = np.multiply(p, np.float32(math.pi), dtype=np.float32)
    return np.divide(prod, np.float32(2.0), dtype=np.float32)
