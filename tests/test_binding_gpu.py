"""The binding on the GPU in a fresh process: the library loaded before torch is imported."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# The library is loaded (set_option) before the script imports torch itself.  torch links the
# HIP runtime under another file name than the library does; the binding imports torch before it
# loads the library so that both use one runtime (otherwise torch's streams and allocations are
# unknown to the library's runtime and the first device call fails).
SCRIPT = """
import rope_ltx3drope_amd as rla
rla.set_option(rla.OPT_PATH, 0)
import torch
q = torch.randn(1, 2, 3, 4, 2, 48, device="cuda:0").to(torch.bfloat16)
k = torch.randn(1, 2, 3, 4, 2, 48, device="cuda:0").to(torch.bfloat16)
qo, ko = rla.forward_pair(q, k, (16, 16, 16))
torch.cuda.synchronize()
s = rla.stats()
print("ok", s["fast_launches"], s["gate_trusted"], flush=True)
"""


def test_library_loaded_before_torch_shares_its_runtime():
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "ok 1 1" in r.stdout, r.stdout


# The C ABI on its own: no torch in the process.  Device memory comes from the HIP runtime the
# library links (hipMalloc through ctypes), the inputs and the expected outputs from files the
# parent wrote (workload 1 and the oracle).
C_ABI_SCRIPT = r"""
import ctypes, sys
import numpy as np
lib_path, data = sys.argv[1], np.load(sys.argv[2])
L = ctypes.CDLL(lib_path)
hip = ctypes.CDLL("libamdhip64.so.7")
vp, i64 = ctypes.c_void_p, ctypes.c_int64
hip.hipMalloc.argtypes = [ctypes.POINTER(vp), ctypes.c_size_t]
hip.hipMemcpy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int]
hip.hipFree.argtypes = [vp]
L.ltx3drope_tables_build.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, ctypes.c_double, vp,
                                     ctypes.POINTER(vp)]
L.ltx3drope_apply_qk.argtypes = [vp, vp, vp, vp, ctypes.c_int] + [i64] * 6 + [vp, vp]
L.ltx3drope_tables_release.argtypes = [vp]
assert "torch" not in sys.modules
q, k = data["q"], data["k"]
nbytes = q.nbytes
bufs = []
for _ in range(4):
    p = vp()
    assert hip.hipMalloc(ctypes.byref(p), nbytes) == 0
    bufs.append(p)
dq, dk, dqo, dko = bufs
assert hip.hipMemcpy(dq, q.ctypes.data, nbytes, 1) == 0 and hip.hipMemcpy(dk, k.ctypes.data, nbytes, 1) == 0
B, T, H, W, heads, D = q.shape
tab = vp()
assert L.ltx3drope_tables_build(0, T, H, W, 16, 16, 16, 10000.0, None, ctypes.byref(tab)) == 0
st = L.ltx3drope_apply_qk(dqo, dko, dq, dk, 0, B, T, H, W, heads, D, tab, None)  # 0: F32
assert st == 0, st
qo, ko = np.empty_like(q), np.empty_like(k)
assert hip.hipMemcpy(qo.ctypes.data, dqo, nbytes, 2) == 0 and hip.hipMemcpy(ko.ctypes.data, dko, nbytes, 2) == 0
assert L.ltx3drope_tables_release(tab) == 0
for p in bufs:
    hip.hipFree(p)
ok = np.array_equal(qo.view(np.uint32), data["want_q"].view(np.uint32)) and \
     np.array_equal(ko.view(np.uint32), data["want_k"].view(np.uint32))
print("ok" if ok else "MISMATCH", flush=True)
"""


def test_c_abi_without_torch(tmp_path):
    """Workload 1 through the C ABI alone (ctypes and the HIP runtime, no torch in the process),
    bit for bit against the oracle."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import oracle
    import workloads
    from rope_ltx3drope_amd import _lib

    w = workloads.WORKLOADS[1]
    (q, k), = workloads.generate(w)
    want_q, want_k = oracle.rope3d_qk(q, k, w.dtype, w.split, w.base)
    assert w.split == (16, 16, 16) and w.dtype == oracle.F32 and _lib.DTYPE_F32 == 0
    data = tmp_path / "w1.npz"
    np.savez(data, q=q, k=k, want_q=want_q, want_k=want_k)
    r = subprocess.run([sys.executable, "-c", C_ABI_SCRIPT, _lib.LIB_PATH, str(data)], cwd=str(tmp_path),
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("ok"), r.stdout
