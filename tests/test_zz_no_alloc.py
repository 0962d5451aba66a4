"""The entry point that allocates no device memory (ltx3drope_apply_qk_noalloc), through the C ABI:
on two calls in a row, the second on a smaller input, its outputs equal ltx3drope_apply_qk's and the
oracle's bit for bit.  The gate verifies every call here, so each call counts its mismatches in the
library's static device scratch: a counter that was not cleared, or not read back, would report a
mismatch and disable the fast kernel, which the test also checks for."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

DEV = "cuda:0"
CALLS = [  # (dtype, shape, split): the second input is smaller than the first
    (oracle.BF16, (1, 4, 16, 16, 16, 128), (32, 48, 48)),
    (oracle.BF16, (1, 2, 4, 6, 4, 64), (16, 24, 24)),
]
CALLS_F32 = [
    (oracle.F32, (2, 3, 8, 8, 8, 96), (32, 32, 32)),
    (oracle.F32, (1, 2, 3, 5, 2, 48), (16, 16, 16)),
]


def log(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    if dtype == oracle.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def raw(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def call(name, dtype, q, k, qo, ko, tab):
    code = _lib.DTYPE_BF16 if dtype == oracle.BF16 else _lib.DTYPE_F32
    stream = torch.cuda.current_stream().cuda_stream
    return getattr(_lib.lib(), name)(qo.data_ptr(), ko.data_ptr(), q.data_ptr(), k.data_ptr(), code, *q.shape,
                                     tab.handle, stream)


@pytest.mark.parametrize("calls", [CALLS, CALLS_F32], ids=["bf16", "f32"])
def test_noalloc_equals_apply_qk_on_two_calls(calls):
    assert torch.cuda.is_available()
    rla.set_option(rla.OPT_PATH, 0)
    rla.set_option(rla.OPT_GATE, 2)  # verify every call
    try:
        for i, (dtype, shape, split) in enumerate(calls):
            log(f"call {i}: {dtype} {shape} split {split}")
            q, k = workloads.generate_custom(shape, dtype, seed=700 + i)
            dq, dk = to_dev(q, dtype), to_dev(k, dtype)
            with rla.tables_build(*shape[1:4], split) as tab:
                ref_q, ref_k = torch.empty_like(dq), torch.empty_like(dk)
                assert call("ltx3drope_apply_qk", dtype, dq, dk, ref_q, ref_k, tab) == _lib.OK
                out_q, out_k = torch.full_like(dq, 7.0), torch.full_like(dk, -7.0)
                torch.cuda.synchronize()
                before = rla.stats()
                assert call("ltx3drope_apply_qk_noalloc", dtype, dq, dk, out_q, out_k, tab) == _lib.OK
                torch.cuda.synchronize()
                after = rla.stats()
            assert after["gate_verifications"] == before["gate_verifications"] + 1
            assert after["gate_disabled"] == 0 and after["fast_launches"] == before["fast_launches"] + 1
            assert torch.equal(raw(out_q), raw(ref_q)) and torch.equal(raw(out_k), raw(ref_k))
            want_q, want_k = oracle.rope3d_qk(q, k, dtype, split)
            for got, want in ((out_q, want_q), (out_k, want_k)):
                host = raw(got).cpu().numpy()
                assert np.array_equal(host.view(np.uint16 if dtype == oracle.BF16 else np.uint32),
                                      want.view(np.uint16 if dtype == oracle.BF16 else np.uint32))
    finally:
        rla.set_option(rla.OPT_GATE, 1)


def test_noalloc_refuses_what_the_precheck_refuses():
    shape, split = (1, 2, 3, 4, 2, 12), (4, 4, 4)
    q = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    with rla.tables_build(2, 3, 5, split) as tab:  # another grid
        st = call("ltx3drope_apply_qk_noalloc", oracle.BF16, q, q.clone(), torch.empty_like(q), torch.empty_like(q),
                  tab)
    assert st == _lib.E_TABLE_MISMATCH
