"""GPU: the DiT frequency-grid kernel against the oracle, bit for bit (float32 output of either
recipe), through the binding and through the C ABI with no torch tensor involved."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle.dit_freqs as df

pytestmark = pytest.mark.gpu

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

DEV = "cuda:0"
CASES = [(10000.0, 4096, 6), (10000.0, 2048, 6), (10000.0, 128, 2), (500.0, 96, 3), (1.0e6, 256, 2),
         (2.5, 64, 1), (10000.0, 11, 6), (0.37, 50, 1), (3.0e38, 40, 1), (1.0, 12, 1),
         (10000.0, 6 * 4097, 6)]


def log(msg):
    print(f"[dit-gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("theta,dim,ne", CASES)
@pytest.mark.parametrize("double", [True, False], ids=["f64", "f32"])
def test_grid_kernel_equals_oracle(theta, dim, ne, double):
    log(f"theta {theta} dim {dim} ne {ne} double {double}")
    got = rla.dit_freq_grid(theta, dim, ne, double, device=DEV)
    torch.cuda.synchronize()
    want = df.freq_grid(theta, dim, ne, double)
    g = got.cpu().numpy().view(np.uint32)
    assert g.shape == want.shape
    bad = np.flatnonzero(g != want.view(np.uint32))
    assert bad.size == 0, (bad[:5], g[bad[:5]], want.view(np.uint32)[bad[:5]])


def test_grid_kernel_through_the_c_abi():
    """Raw device memory from the library's own allocator-free path: a torch buffer is used only as
    memory, the call is made with plain pointers, on a side stream, with a guard band after the
    grid that must stay untouched."""
    L = _lib.lib()
    n = 4096 // 6
    buf = torch.full((n + 64,), -3.0, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    cnt = ctypes.c_int64(-1)
    torch.cuda.synchronize()
    assert L.ltx3drope_dit_freq_grid(10000.0, 4096, 6, 1, buf.data_ptr(), s.cuda_stream, ctypes.byref(cnt)) == _lib.OK
    s.synchronize()
    assert cnt.value == n
    np.testing.assert_array_equal(buf[:n].cpu().numpy().view(np.uint32),
                                  df.freq_grid(10000.0, 4096, 6, True).view(np.uint32))
    assert bool((buf[n:] == -3.0).all())
    # an allocation too small for the grid, and host memory, are refused before any launch: 2^22
    # values (16 MiB) do not fit in the 2 MiB small-block segment of torch's allocator that holds
    # an 8-float tensor (the library sees allocations, not tensors)
    small = torch.empty(8, dtype=torch.float32, device=DEV)
    assert L.ltx3drope_dit_freq_grid(10000.0, 1 << 22, 1, 1, small.data_ptr(), None, None) == _lib.E_UNSUPPORTED
    host = torch.empty(n, dtype=torch.float32).pin_memory()
    assert L.ltx3drope_dit_freq_grid(10000.0, 4096, 6, 1, host.data_ptr(), None, None) == _lib.E_UNSUPPORTED
    torch.cuda.synchronize()


def test_grid_kernel_repeated_calls_identical():
    a = rla.dit_freq_grid(10000.0, 4096, 6, False, device=DEV)
    b = rla.dit_freq_grid(10000.0, 4096, 6, False, device=DEV)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    e = rla.dit_freq_grid(10000.0, 5, 6, True, device=DEV)
    assert e.numel() == 0
