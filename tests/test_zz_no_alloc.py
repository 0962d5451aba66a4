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


def test_noalloc_verifications_from_threads_share_the_scratch_safely():
    """Four host threads, each on its own stream, call the no-allocation entry point three times on
    configurations of their own with every call verified: all verifications count in the one static
    scratch counter, which the library hands to one verification at a time, so none may see
    another's count (a stray count would disable the fast kernel) and every output equals the
    oracle's."""
    import threading

    cases = [((1, 2, 4, 4, 8, 64), (16, 24, 24)), ((1, 3, 4, 6, 4, 96), (32, 32, 32)),
             ((2, 2, 3, 5, 6, 64), (16, 16, 32)), ((1, 4, 2, 8, 8, 128), (32, 48, 48))]
    inputs = [workloads.generate_custom(shape, oracle.BF16, seed=900 + i) for i, (shape, _) in enumerate(cases)]
    dev_in = [(to_dev(q, oracle.BF16), to_dev(k, oracle.BF16)) for q, k in inputs]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    results, errors = [None] * len(cases), []
    start = threading.Barrier(len(cases))
    rla.set_option(rla.OPT_PATH, 0)
    rla.set_option(rla.OPT_GATE, 2)  # verify every call
    before = rla.stats()

    def worker(i):
        try:
            shape, split = cases[i]
            dq, dk = dev_in[i]
            with rla.tables_build(*shape[1:4], split) as tab:
                start.wait(timeout=60)
                outs = []
                with torch.cuda.stream(streams[i]):
                    for _ in range(3):
                        qo, ko = torch.empty_like(dq), torch.empty_like(dk)
                        rla.apply_qk_noalloc(dq, dk, tab, qo, ko, stream=streams[i])
                        outs.append((qo, ko))
                streams[i].synchronize()
            results[i] = outs
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    try:
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
    finally:
        rla.set_option(rla.OPT_GATE, 1)
    assert not errors, errors
    after = rla.stats()
    assert after["gate_verifications"] == before["gate_verifications"] + 3 * len(cases)
    assert after["gate_disabled"] == before["gate_disabled"]
    for i, (shape, split) in enumerate(cases):
        want_q, want_k = oracle.rope3d_qk(*inputs[i], oracle.BF16, split)
        for qo, ko in results[i]:
            for got, want in ((qo, want_q), (ko, want_k)):
                assert np.array_equal(raw(got).cpu().numpy().view(np.uint16), want.view(np.uint16)), (i, shape)
