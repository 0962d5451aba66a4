"""GPU parity of the rotate-half RoPE (through the C ABI) against oracle.neox, 0 ULP."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.neox as nx
import workloads
from tests.oracle_full import compare_full_neox

pytestmark = pytest.mark.gpu

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

DEV = "cuda:0"


def log(msg):
    print(f"[neox-gpu] {msg}", flush=True)


@pytest.fixture(autouse=True)
def fresh():
    assert torch.cuda.is_available()
    _lib.lib()
    rla.set_option(rla.OPT_PATH, 0)
    rla.stats_reset()
    rla.neox_position_errors(0, reset=True)
    yield
    rla.set_option(rla.OPT_PATH, 0)
    torch.cuda.synchronize()


def to_dev(x, dtype):
    if dtype == oracle.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_host(t, dtype):
    if dtype == oracle.BF16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def assert_bitexact(got, want, dtype, what):
    """Raw bits (NaN outputs are the canonical quiet NaN on both sides)."""
    g = got.view(np.uint32 if dtype == oracle.F32 else np.uint16)
    w = want.view(np.uint32 if dtype == oracle.F32 else np.uint16)
    neq = g != w
    n = int(neq.sum())
    assert n == 0, f"{what}: {n} mismatching elements, first at {np.argwhere(neq)[:3].tolist()}"


def run(w, path, q=None, k=None, pos=None, cache=None, inplace=False):
    if q is None:
        q, k, pos, cache = workloads.generate_neox(w)
    rla.set_option(rla.OPT_PATH, path)
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    dpos = torch.from_numpy(pos).to(DEV)
    dcache = to_dev(cache, w.cache_dtype)
    qo, ko = rla.neox_apply_qk(dq, dk, dpos, dcache, inplace=inplace)
    torch.cuda.synchronize()
    if inplace:
        assert qo.data_ptr() == dq.data_ptr() and ko.data_ptr() == dk.data_ptr()
    return (q, k, pos, cache), to_host(qo, w.dtype), to_host(ko, w.dtype)


CASES = ["n1", "n2", "n3"]


@pytest.mark.parametrize("key", CASES)
@pytest.mark.parametrize("path", [0, 2], ids=["fast", "plain"])
def test_workloads_full(key, path):
    w = workloads.NEOX_WORKLOADS[key]
    log(f"{w.key} path {path}")
    (q, k, pos, cache), gq, gk = run(w, path)
    assert_bitexact(gq, nx.neox_rope(q, w.dtype, pos, cache, w.cache_dtype), w.dtype, "q")
    assert_bitexact(gk, nx.neox_rope(k, w.dtype, pos, cache, w.cache_dtype), w.dtype, "k")
    s = rla.stats()
    if path == 2:
        assert s["plain_launches"] == 1 and s["fast_launches"] == 0
    else:
        assert s["fast_launches"] == 1


SHAPES = [
    # dtype, tokens, q_heads, k_heads, D, max_pos, cache dtype  (plain-only shapes included)
    (oracle.BF16, 37, 5, 1, 32, 64, oracle.F32),
    (oracle.BF16, 13, 2, 3, 48, 20, oracle.BF16),
    (oracle.BF16, 9, 3, 2, 20, 30, oracle.F32),   # half row of 10 bf16: not whole 16-byte vectors
    (oracle.F32, 21, 4, 4, 8, 40, oracle.F32),
    (oracle.F32, 17, 2, 1, 16, 9, oracle.BF16),
    (oracle.F32, 5, 1, 1, 2, 3, oracle.F32),
    (oracle.BF16, 300, 16, 8, 256, 512, oracle.BF16),
    # more head rows per lane than one batch of four: 3 and 2 batches, the last partial
    (oracle.BF16, 50, 40, 24, 256, 100, oracle.F32),
    (oracle.F32, 33, 12, 5, 256, 64, oracle.BF16),   # 2 head slots per wavefront, uneven K rows
    (oracle.BF16, 11, 100, 7, 48, 20, oracle.BF16),  # 21 head slots, one lane idle
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
@pytest.mark.parametrize("inplace", [False, True], ids=["fresh", "inplace"])
def test_shapes_full(shape, inplace):
    dtype, tokens, qh, kh, D, maxp, cdt = shape
    w = workloads.NeoxWorkload("s", dtype, tokens, qh, kh, D, maxp, cdt, "random", tokens + D)
    (q, k, pos, cache), gq, gk = run(w, 0, inplace=inplace)
    assert_bitexact(gq, nx.neox_rope(q, dtype, pos, cache, cdt), dtype, "q")
    assert_bitexact(gk, nx.neox_rope(k, dtype, pos, cache, cdt), dtype, "k")


def test_out_of_range_positions_are_flagged_not_read():
    w = workloads.NEOX_WORKLOADS["n3"]
    q, k, pos, cache = workloads.generate_neox(w)
    bad = pos.copy()
    bad[[3, 10, 11]] = [-1, w.max_position, 1 << 40]
    for path in (0, 2):
        rla.neox_position_errors(0, reset=True)
        _, gq, gk = run(w, path, q, k, bad, cache)
        assert rla.neox_position_errors(0, reset=True) == 6  # 3 tokens x (Q, K)
        good = np.ones(len(pos), bool)
        good[[3, 10, 11]] = False
        want_q = nx.neox_rope(q[good], w.dtype, pos[good], cache, w.cache_dtype)
        assert_bitexact(gq[good], want_q, w.dtype, "q on valid tokens")
        canon = np.uint32(0x7FC00000) if w.dtype == oracle.F32 else np.uint16(0x7FC0)
        raw = (lambda a: a.view(np.uint32)) if w.dtype == oracle.F32 else (lambda a: a)
        assert (raw(gq[~good]) == canon).all() and (raw(gk[~good]) == canon).all()


def test_full_size_every_element_and_fast_equals_plain():
    """The 32k-token workload: both kernels equal, and every element of Q' and K' equals the
    oracle's."""
    w = workloads.NEOX_WORKLOADS["n4"]
    log("n4: generating inputs")
    q, k, pos, cache = workloads.generate_neox(w)
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    dpos, dcache = torch.from_numpy(pos).to(DEV), to_dev(cache, w.cache_dtype)
    fq, fk = rla.neox_apply_qk(dq, dk, dpos, dcache)
    rla.set_option(rla.OPT_PATH, 2)
    pq, pk = rla.neox_apply_qk(dq, dk, dpos, dcache)
    torch.cuda.synchronize()
    assert torch.equal(fq.view(torch.int16), pq.view(torch.int16))
    assert torch.equal(fk.view(torch.int16), pk.view(torch.int16))
    for name, x, out in (("q", q, fq), ("k", k, fk)):
        log(f"n4: comparing every element of {name} with the oracle")
        n, first = compare_full_neox(x, to_host(out, w.dtype), w.dtype, pos, cache, w.cache_dtype)
        assert n == 0, f"{name}: {n} mismatching elements of {x.size}, first {first}"


def test_precheck_refusals_on_device():
    w = workloads.NEOX_WORKLOADS["n1"]
    q, k, pos, cache = workloads.generate_neox(w)
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    dpos, dcache = torch.from_numpy(pos).to(DEV), to_dev(cache, w.cache_dtype)
    before = torch.cuda.memory_allocated(DEV)
    assert rla.neox_can_use(dq, dk, dpos, dcache) == (True, "OK")
    assert torch.cuda.memory_allocated(DEV) == before  # the query allocates nothing
    qo, ko = torch.empty_like(dq), torch.empty_like(dk)
    assert rla.neox_can_use(dq, dk, dpos, dcache, qo, ko) == (True, "OK")
    assert rla.neox_can_use(dq, dk, dpos, dcache, dq, dk) == (True, "OK")  # exact in-place aliasing
    with pytest.raises(ValueError):
        rla.neox_can_use(dq, dk, dpos, dcache, qo, None)
    assert rla.neox_can_use(dq, dk, dpos.int(), dcache)[0] is False
    assert rla.neox_can_use(dq, dk, dpos.cpu(), dcache) == (False, "NOT_DEVICE_PTR")
    with pytest.raises(rla.Ltx3dRopeUnsupported):
        rla.neox_apply_qk(dq, dk, dpos, dcache[:, :8])
    with pytest.raises(rla.Ltx3dRopeUnsupported):
        rla.neox_apply_qk(dq[:, :, :15].contiguous(), dk[:, :, :15].contiguous(), dpos, dcache[:, :15].contiguous())
    assert rla.stats()["fast_launches"] == 0 and rla.stats()["plain_launches"] == 0


def test_zero_tokens():
    """An empty token batch: empty outputs, nothing launched, no position error counted."""
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    pos = torch.empty(0, dtype=torch.int64, device=DEV)
    cache = torch.zeros((16, 64), dtype=torch.float32, device=DEV)
    assert rla.neox_can_use(q, k, pos, cache) == (True, "OK")
    qo, ko = rla.neox_apply_qk(q, k, pos, cache)
    assert qo.shape == q.shape and ko.shape == k.shape
    assert rla.stats()["fast_launches"] == 0 and rla.stats()["plain_launches"] == 0
    assert rla.neox_position_errors(0) == 0


@pytest.mark.parametrize("seed", [11, 22])
def test_random_configurations(seed):
    """Twenty seeded random configurations per seed (head_dim, head counts, dtypes, cache sizes; half
    of the head dims give whole 16-byte half rows), fast and plain kernels, against the oracle."""
    rng = np.random.default_rng(seed)
    for i in range(20):
        dtype = oracle.BF16 if rng.random() < 0.6 else oracle.F32
        cdt = oracle.BF16 if rng.random() < 0.5 else oracle.F32
        es = 2 if dtype == oracle.BF16 else 4
        unit = 2 * (16 // es) if rng.random() < 0.5 else 2  # whole 16-byte half rows, or any even D
        D = int(unit * rng.integers(1, 256 // unit + 1))
        w = workloads.NeoxWorkload("r", dtype, int(rng.integers(1, 300)), int(rng.integers(1, 21)),
                                   int(rng.integers(1, 13)), D, int(rng.integers(1, 600)), cdt, "random",
                                   seed * 100 + i)
        log(f"random {w}")
        inputs = workloads.generate_neox(w)
        for path in (0, 2):
            (q, k, pos, cache), gq, gk = run(w, path, *inputs)
            assert_bitexact(gq, nx.neox_rope(q, dtype, pos, cache, cdt), dtype, f"q {w} path {path}")
            assert_bitexact(gk, nx.neox_rope(k, dtype, pos, cache, cdt), dtype, f"k {w} path {path}")
    assert rla.neox_position_errors(0) == 0


def test_more_tokens_than_the_fast_grid_holds_use_the_plain_kernel():
    """2^25 + 3 tokens of one head of 16 bf16 values: two 64-lane workgroups per token would need
    2^32 work-items or more, so the call runs on the plain kernel; every element against the
    oracle.  Inputs are drawn on the device (workloads.generate_neox_device)."""
    tokens, D, maxp = (1 << 25) + 3, 16, 1000
    log("2^25 + 3 tokens: generating inputs on the device")
    dq, dk, dpos = workloads.generate_neox_device(tokens, 1, 1, D, maxp, 2024, DEV)
    w = workloads.NeoxWorkload("big", oracle.BF16, 16, 1, 1, D, maxp, oracle.F32, "random", 31)
    _, _, _, cache = workloads.generate_neox(w)
    qo, ko = rla.neox_apply_qk(dq, dk, dpos, to_dev(cache, oracle.F32))
    torch.cuda.synchronize()
    s = rla.stats()
    assert s["plain_launches"] == 1 and s["fast_launches"] == 0
    assert rla.neox_position_errors(0) == 0
    pos = dpos.cpu().numpy()
    for name, x, out in (("q", dq, qo), ("k", dk, ko)):
        log(f"2^25 + 3 tokens: comparing every element of {name} with the oracle")
        n, first = compare_full_neox(to_host(x, oracle.BF16), to_host(out, oracle.BF16), oracle.BF16, pos, cache,
                                     oracle.F32)
        assert n == 0, f"{name}: {n} mismatching elements, first {first}"


def test_tensors_of_more_than_2_to_the_31_elements():
    """2^23 tokens of one query and one KV head of head_dim 384 in bf16: 3,221,225,472 elements per
    tensor (between 2^31 and 2^32, 6.4 GB), drawn on the device.  The fast kernel against the plain
    kernel over the whole output, and every element against the oracle."""
    tokens, D, maxp = 1 << 23, 384, 4096
    log("2^23 tokens x 384: generating inputs on the device")
    dq, dk, dpos = workloads.generate_neox_device(tokens, 1, 1, D, maxp, 77, DEV)
    w = workloads.NeoxWorkload("big", oracle.BF16, 16, 1, 1, D, maxp, oracle.BF16, "random", 33)
    _, _, _, cache = workloads.generate_neox(w)
    dcache = to_dev(cache, oracle.BF16)
    fq, fk = rla.neox_apply_qk(dq, dk, dpos, dcache)
    rla.set_option(rla.OPT_PATH, 2)
    pq, pk = rla.neox_apply_qk(dq, dk, dpos, dcache)
    torch.cuda.synchronize()
    s = rla.stats()
    assert s["fast_launches"] == 1 and s["plain_launches"] == 1
    assert torch.equal(fq.view(torch.int16), pq.view(torch.int16))
    assert torch.equal(fk.view(torch.int16), pk.view(torch.int16))
    del pq, pk
    pos = dpos.cpu().numpy()
    for name, x, out in (("q", dq, fq), ("k", dk, fk)):
        log(f"2^23 tokens x 384: comparing every element of {name} with the oracle")
        n, first = compare_full_neox(to_host(x, oracle.BF16), to_host(out, oracle.BF16), oracle.BF16, pos, cache,
                                     oracle.BF16)
        assert n == 0, f"{name}: {n} mismatching elements, first {first}"
    assert rla.neox_position_errors(0) == 0


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.F32])
@pytest.mark.parametrize("path", [0, 2], ids=["fast", "plain"])
def test_special_values_raw_bits(dtype, path):
    """NaNs of several signs and payloads, infinities, zeros, huge and tiny values in Q and K: every
    output equals the oracle's raw bits, NaN results being the canonical quiet NaN."""
    w = workloads.NeoxWorkload("sv", dtype, 40, 4, 2, 64, 64, oracle.F32, "random", 91)
    q, k, pos, cache = workloads.generate_neox(w)
    rng = np.random.Generator(np.random.PCG64(92))
    if dtype == oracle.F32:
        special = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF812345, 0x7F800000, 0xFF800000, 0x80000000,
                            0x00000001, 0x7F7FFFFF], np.uint32).view(np.float32)
    else:
        special = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFF92, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x7F7F], np.uint16)
    for x in (q, k):
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, flat.size // 8, replace=False)
        flat[idx] = special[rng.integers(0, len(special), idx.size)]
    _, gq, gk = run(w, path, q, k, pos, cache)
    assert_bitexact(gq, nx.neox_rope(q, dtype, pos, cache, oracle.F32), dtype, "q")
    assert_bitexact(gk, nx.neox_rope(k, dtype, pos, cache, oracle.F32), dtype, "k")
