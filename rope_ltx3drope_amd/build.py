"""Build libltx3drope.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m rope_ltx3drope_amd.build          # or: python rope_ltx3drope_amd/build.py

Every source is compiled on each call; objects go to rope_ltx3drope_amd/_build/.
Floating-point contraction is off everywhere (the rotation must not fuse its
products into FMAs and the host tables are plain float64 libm results), and
hipcc's automatic packed-fp32 instructions are disabled on the device side.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libltx3drope.so")
ARCH = os.environ.get("LTX3DROPE_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-ffp-contract=off", "-fno-fast-math",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
DEVICE = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
]
SOURCES = [  # (file, language, extra flags)
    ("kernels.hip", "hip", DEVICE),
    ("plain.hip", "hip", DEVICE),
    ("neox.hip", "hip", DEVICE),
    ("patchify.hip", "hip", DEVICE),
    ("dit_freqs.hip", "hip", DEVICE),
    ("api.cpp", "c++", ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]),
    ("tables.cpp", "c++", ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-fno-builtin"]),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src, lang, extra in SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-x", lang, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + extra
        if save_temps and src.endswith(".hip"):
            cmd += ["--save-temps"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=OUT_DIR)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + ["-Wl,-soname,libltx3drope.so"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=OUT_DIR)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))
