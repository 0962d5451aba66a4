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
