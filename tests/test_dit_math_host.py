"""CPU test of the DiT frequency kernel's arithmetic (rope_ltx3drope_amd/csrc/dit_math.h), built for
the host with g++ (the same IEEE operations as on the device, contraction off), against the oracle:
the whole grid bit for bit for the float64 and float32 recipes, the correctly rounded power on
random bases and exponents in both precisions, and the ln 2 constant against a 60-digit value.
The device build of the same source is compared with the oracle by tests/test_dit_freqs_gpu.py."""
from __future__ import annotations

import os
import shutil
import subprocess
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle.dit_freqs as df

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rope_ltx3drope_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host_sanitize", "dit_math_check.cpp")
CASES = [(10000.0, 4096, 6), (10000.0, 2048, 6), (10000.0, 128, 2), (500.0, 96, 3), (1.0e6, 256, 2),
         (2.5, 64, 1), (10000.0, 11, 6), (10000.0, 5, 6), (0.37, 50, 1), (3.0e38, 40, 1), (1.0, 12, 1),
         (10000.0, 6 * 4097, 6)]


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    out = tmp_path_factory.mktemp("dit") / "dit_math_check"
    cmd = [gxx, "-O2", "-std=c++20", "-ffp-contract=off", "-fno-fast-math", "-D__host__=", "-D__device__=",
           "-I" + CSRC, SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(out)


@pytest.mark.parametrize("theta,dim,ne", CASES)
@pytest.mark.parametrize("double", [True, False], ids=["f64", "f32"])
def test_host_build_grid_equals_oracle(exe, theta, dim, ne, double):
    r = subprocess.run([exe, "grid", repr(theta), str(dim), str(ne), "1" if double else "0"], capture_output=True,
                       text=True, timeout=120, check=True)
    got = np.array([int(h, 16) for h in r.stdout.split()], dtype=np.uint32)
    want = df.freq_grid(theta, dim, ne, double).view(np.uint32)
    assert got.shape == want.shape
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (bad[:5], got[bad[:5]], want[bad[:5]])


def test_host_build_pow_is_correctly_rounded(exe):
    rng = np.random.default_rng(2024)
    cases = []
    for _ in range(1500):
        double = bool(rng.integers(0, 2))
        base = float(np.exp(rng.uniform(np.log(1e-3), np.log(1e30))))
        x = float(rng.uniform(0.0, 1.0))
        if not double:
            base, x = float(np.float32(base)), float(np.float32(x))
        cases.append((base, x, double))
    cases += [(10000.0, 0.5, True), (4.0, 0.5, True), (3.0, 2.0, True), (10000.0, 1.0, False), (2.0, 0.0, True)]
    inp = "".join(f"{np.float64(b).view(np.uint64):x} {np.float64(x).view(np.uint64):x} {int(d)}\n"
                  for b, x, d in cases)
    r = subprocess.run([exe, "pow"], input=inp, capture_output=True, text=True, timeout=300, check=True)
    outs = r.stdout.split()
    assert len(outs) == len(cases)
    bad = []
    for (b, x, d), h in zip(cases, outs):
        want = df.pow_rn(b, x, d)
        got = int(h, 16)
        want_bits = int(np.array(want, np.float64 if d else np.float32).view(np.uint64 if d else np.uint32))
        if got != want_bits:
            bad.append((b, x, d, hex(got), hex(want_bits)))
    assert not bad, bad[:5]


def test_ln2_constant(exe):
    r = subprocess.run([exe, "ln2"], capture_output=True, text=True, timeout=60, check=True)
    hi, lo = (np.uint64(int(h, 16)).view(np.float64) for h in r.stdout.split())
    with localcontext() as ctx:
        ctx.prec = 60
        ln2 = Fraction(Decimal(2).ln())
    assert float(hi) == float(ln2)  # the double nearest ln 2
    assert float(lo) == float(ln2 - Fraction(float(hi)))  # the double nearest the rest


def test_host_build_pow_wide_random_sweep(exe):
    """20000 seeded random powers over a wider domain (bases from 1e-30 to 1e38, one exponent in
    five in [-2, 2]) in both precisions: every result equals the correctly rounded power.  Cases the
    oracle cannot decide (a result outside the format's range, or within its evaluation's error of a
    rounding boundary) are skipped; they are fewer than 1 %."""
    rng = np.random.default_rng(77)
    cases = []
    for _ in range(20000):
        double = bool(rng.integers(0, 2))
        base = float(np.exp(rng.uniform(np.log(1e-30), np.log(1e38))))
        x = float(rng.uniform(0.0, 1.0)) if rng.random() < 0.8 else float(rng.uniform(-2.0, 2.0))
        if not double:
            base, x = float(np.float32(base)), float(np.float32(x))
        cases.append((base, x, double))
    inp = "".join(f"{np.float64(b).view(np.uint64):x} {np.float64(x).view(np.uint64):x} {int(d)}\n"
                  for b, x, d in cases)
    r = subprocess.run([exe, "pow"], input=inp, capture_output=True, text=True, timeout=300, check=True)
    outs = r.stdout.split()
    assert len(outs) == len(cases)
    bad, skipped = [], 0
    for (b, x, d), h in zip(cases, outs):
        try:
            want = df.pow_rn(b, x, d)
        except (ArithmeticError, OverflowError, ValueError):
            skipped += 1
            continue
        want_bits = int(np.array(want, np.float64 if d else np.float32).view(np.uint64 if d else np.uint32))
        if int(h, 16) != want_bits:
            bad.append((b, x, d, h, hex(want_bits)))
    assert not bad, bad[:5]
    assert skipped < len(cases) // 100
