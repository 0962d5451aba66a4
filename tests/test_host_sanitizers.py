"""The library's host code under AddressSanitizer + UndefinedBehaviorSanitizer and under
ThreadSanitizer (CPU only).

api.cpp and tables.cpp are compiled for the host with clang and the sanitizer, linked with
stand-ins for the HIP runtime and the kernel launchers (tests/host_sanitize/stubs.cpp), and
driven by tests/host_sanitize/driver.cpp: eight threads build, read, hold and release table
sets of 24 grids through the 16-entry cache (evictions while handles are held), run the
precheck, refused launches, statistics, cache clears and the DiT frequency grid, all in
host-table mode.  At the end every table must be freed and no HIP stand-in called.  Then,
against stand-ins that emulate a device 0 with host memory, injected hipMalloc failures must
give E_NOMEM (out of memory) or E_HIP (another error) from the table upload and the device
counter's allocation, leave no table or allocation behind, and a later build must succeed.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = [os.path.join(ROOT, "rope_ltx3drope_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "rope_ltx3drope_amd", "csrc", "tables.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "stubs.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")]

pytestmark = pytest.mark.skipif(not shutil.which(CLANG), reason="clang++ of the ROCm toolchain not found")


@pytest.mark.parametrize("sanitizer,iters", [("address,undefined", 2000), ("thread", 1000)],
                         ids=["asan_ubsan", "tsan"])
def test_host_code_under_sanitizer(tmp_path, sanitizer, iters):
    exe = tmp_path / "driver"
    cmd = [CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           f"-fsanitize={sanitizer}", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "rope_ltx3drope_amd", "csrc"), *SOURCES, "-o", str(exe), "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe), "8", str(iters)], capture_output=True, text=True, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "host sanitizer driver" in run.stdout


def test_fast_division_matches_hardware_division(tmp_path):
    """fastdiv.h (the kernels' division by invariant divisors) against the hardware division:
    sampled dividends for every divisor up to 2^16 and 200000 random ones, every dividend for two."""
    gxx = shutil.which("g++") or CLANG
    exe = tmp_path / "fastdiv_check"
    src = os.path.join(ROOT, "tests", "host_sanitize", "fastdiv_check.cpp")
    build = subprocess.run([gxx, "-O2", "-std=c++17", "-I" + os.path.join(ROOT, "rope_ltx3drope_amd", "csrc"), src,
                            "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 differ" in run.stdout
