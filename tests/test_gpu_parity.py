"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for bit.

Tolerance is 0 ULP on the raw bits of every element (NaN results are the
canonical quiet NaN on both sides).  Every output is compared element by element
with the oracle: small, ragged and random shapes, and the full-size workloads
(the oracle runs over blocks of each frame in a thread pool, tests/oracle_full.py),
up to the largest tensors the op takes.  Properties that hold at any size are
checked besides: fast kernel == plain kernel on the whole output, unit-vector
readback of the tables, untouched inputs and guard bands.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import oracle_full

pytestmark = pytest.mark.gpu

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

DEV = "cuda:0"


def log(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _lib.lib()  # fails loudly if the HIP library is missing
    yield


@pytest.fixture(autouse=True)
def fresh_state():
    for opt, v in ((rla.OPT_PATH, 0), (rla.OPT_GATE, 1), (rla.OPT_FORCE_GATE_MISMATCH, 0), (rla.OPT_HOST_TABLES, 0)):
        rla.set_option(opt, v)
    rla.gate_reset()
    rla.cache_clear()
    rla.stats_reset()
    yield
    rla.set_option(rla.OPT_PATH, 0)
    rla.set_option(rla.OPT_FORCE_GATE_MISMATCH, 0)
    torch.cuda.synchronize()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == oracle.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == oracle.BF16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32) if x.dtype == np.float32 else x.view(np.uint16)


def assert_bitexact(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g, w = bits(got), bits(want)
    neq = g != w
    n = int(neq.sum())
    if n:
        idx = np.argwhere(neq)[:5]
        raise AssertionError(f"{what}: {n} mismatching elements, first at {idx.tolist()}: "
                             f"got {[hex(int(g[tuple(i)])) for i in idx]} want {[hex(int(w[tuple(i)])) for i in idx]}")


def run(q, k, split, base=10000.0, path=0):
    rla.set_option(rla.OPT_PATH, path)
    with rla.tables_build(*q.shape[1:4], split, base) as tab:
        qo, ko = rla.apply_qk(q, k, tab)
    torch.cuda.synchronize()
    return qo, ko


# ---------------------------------------------------------------------------
# full element-by-element comparisons
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wk", [1, 2])
@pytest.mark.parametrize("path", [0, 1, 2], ids=["auto", "fast", "plain"])
def test_small_workloads_full(wk, path):
    w = workloads.WORKLOADS[wk]
    log(f"workload {wk} path {path}")
    (q, k), = workloads.generate(w)
    want_q, want_k = oracle.rope3d_qk(q, k, w.dtype, w.split, w.base)
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    qo, ko = run(dq, dk, w.split, w.base, path)
    assert qo.data_ptr() != dq.data_ptr() and ko.data_ptr() != dk.data_ptr()
    assert_bitexact(to_host(qo, w.dtype), want_q, w.dtype, "q")
    assert_bitexact(to_host(ko, w.dtype), want_k, w.dtype, "k")
    # inputs untouched
    assert_bitexact(to_host(dq, w.dtype), q, w.dtype, "q input")
    assert_bitexact(to_host(dk, w.dtype), k, w.dtype, "k input")
    s = rla.stats()
    if path == 1:
        assert s["fast_launches"] == 1 and s["plain_launches"] == 0
    if path == 2:
        assert s["plain_launches"] == 1 and s["fast_launches"] == 0
    if path == 0:
        assert s["gate_verifications"] == 1 and s["gate_trusted"] == 1


RAGGED = [
    # shape, split, dtype  (fast-eligible and plain-only, ragged grids, odd heads)
    ((1, 3, 5, 7, 3, 24), (8, 8, 8), oracle.BF16),
    ((2, 3, 5, 7, 3, 24), (8, 8, 8), oracle.F32),
    ((2, 1, 1, 1, 1, 6), (2, 2, 2), oracle.BF16),
    ((1, 2, 3, 4, 5, 12), (2, 6, 4), oracle.BF16),
    ((1, 5, 3, 2, 7, 40), (8, 16, 16), oracle.BF16),
    ((1, 4, 9, 11, 33, 48), (16, 16, 16), oracle.BF16),
    ((2, 2, 6, 5, 4, 96), (32, 32, 32), oracle.BF16),
    ((1, 3, 4, 5, 2, 128), (32, 48, 48), oracle.F32),
    ((1, 2, 3, 3, 64, 64), (16, 24, 24), oracle.BF16),
    ((1, 2, 2, 2, 17, 16), (4, 4, 8), oracle.F32),
    ((3, 1, 7, 1, 8, 16), (8, 4, 4), oracle.BF16),
    ((1, 9, 1, 13, 2, 12), (4, 4, 4), oracle.F32),
    ((1, 2, 3, 4, 40, 128), (32, 48, 48), oracle.BF16),   # 640 vectors per token
    ((1, 2, 2, 3, 80, 96), (32, 32, 32), oracle.BF16),    # 960 vectors per token
    ((1, 1, 2, 2, 3, 20), (8, 8, 4), oracle.BF16),        # head row not a whole 16-byte vector
    # splits whose chunks are not whole vectors, one token per wavefront: the LDS-assembled table row
    ((1, 2, 3, 4, 16, 96), (30, 34, 32), oracle.BF16),
    ((1, 3, 2, 5, 24, 128), (40, 44, 44), oracle.BF16),
    ((1, 2, 3, 3, 32, 48), (14, 18, 16), oracle.F32),
    ((1, 2, 2, 3, 4, 256), (86, 86, 84), oracle.BF16),    # 128 pairs: two per lane
    ((2, 2, 1, 3, 2, 1024), (342, 342, 340), oracle.BF16),  # the largest row the LDS holds (4 KB)
    ((1, 1, 2, 2, 32, 1040), (346, 348, 346), oracle.BF16),  # larger: per-pair table loads
    ((1, 1, 2, 2, 16, 1056), (352, 352, 352), oracle.BF16),  # larger, whole vectors: direct 16-byte loads
]


@pytest.mark.parametrize("shape,split,dtype", RAGGED, ids=[f"{s}-{sp}-{d}" for s, sp, d in RAGGED])
@pytest.mark.parametrize("path", [1, 2], ids=["fast", "plain"])
def test_ragged_shapes_full(shape, split, dtype, path):
    log(f"ragged {shape} {split} {dtype} path {path}")
    q, k = workloads.generate_custom(shape, dtype, seed=sum(shape) + path)
    want_q, want_k = oracle.rope3d_qk(q, k, dtype, split)
    qo, ko = run(to_dev(q, dtype), to_dev(k, dtype), split, path=path)
    assert_bitexact(to_host(qo, dtype), want_q, dtype, "q")
    assert_bitexact(to_host(ko, dtype), want_k, dtype, "k")


def _random_configs(n, seed):
    """Seeded random shapes, splits, bases and shard placements: half of the splits are multiples of
    the fast kernel's vector width, half are any even widths."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = oracle.BF16 if rng.random() < 0.6 else oracle.F32
        step = (8 if dtype == oracle.BF16 else 4) if rng.random() < 0.5 else 2
        split = tuple(int(step * rng.integers(1, 48 // step + 1)) for _ in range(3))
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 7)), int(rng.integers(1, 7)), int(rng.integers(1, 7)),
                 int(rng.integers(1, 9)), sum(split))
        base = float(rng.choice([10000.0, 500.0, 1.0e6, 2.5]))
        offsets = (0, 0, 0) if rng.random() < 0.5 else tuple(int(x) for x in rng.integers(0, 4, 3))
        out.append((shape, split, dtype, base, offsets))
    return out


@pytest.mark.parametrize("seed", [101, 202, 303])
def test_random_configurations(seed):
    """Sixteen random configurations per seed, each through the gate (auto path) and the plain kernel,
    element by element against the oracle (shards of a larger grid included)."""
    for shape, split, dtype, base, offsets in _random_configs(16, seed):
        log(f"random {shape} {split} {dtype} base {base} offsets {offsets}")
        q, k = workloads.generate_custom(shape, dtype, seed=seed + sum(shape))
        grid = tuple(n + o for n, o in zip(shape[1:4], offsets))
        want_q, want_k = oracle.rope3d_qk(q, k, dtype, split, base, offsets=offsets, grid=grid)
        dq, dk = to_dev(q, dtype), to_dev(k, dtype)
        for path in (0, 2):
            rla.set_option(rla.OPT_PATH, path)
            qo, ko = rla.forward_pair(dq, dk, split, base, grid=grid,
                                      offsets=None if offsets == (0, 0, 0) else offsets)
            torch.cuda.synchronize()
            assert_bitexact(to_host(qo, dtype), want_q, dtype, f"q {shape} {split} path {path}")
            assert_bitexact(to_host(ko, dtype), want_k, dtype, f"k {shape} {split} path {path}")
    assert rla.stats()["gate_disabled"] == 0


def _random_wide_configs(n, seed):
    """Seeded random configurations with wide token rows (up to 40 heads, head_dim up to 192) on
    small grids: rows of whole wavefronts (one decode per wavefront, the token's table row in LDS),
    rows of 32+ vectors that span tokens, and short rows, with aligned and arbitrary even splits."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = oracle.BF16 if rng.random() < 0.6 else oracle.F32
        step = (8 if dtype == oracle.BF16 else 4) if rng.random() < 0.5 else 2
        split = tuple(int(step * rng.integers(1, 64 // step + 1)) for _ in range(3))
        heads = int(rng.choice([1, 3, 4, 8, 12, 16, 24, 32, 40]))
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 5)),
                 heads, sum(split))
        offsets = (0, 0, 0) if rng.random() < 0.6 else tuple(int(x) for x in rng.integers(0, 3, 3))
        out.append((shape, split, dtype, offsets))
    return out


@pytest.mark.parametrize("seed", [404, 505])
def test_random_wide_rows(seed):
    """Twelve wide-row random configurations per seed, through the gate and the plain kernel,
    element by element against the oracle."""
    for shape, split, dtype, offsets in _random_wide_configs(12, seed):
        log(f"wide {shape} {split} {dtype} offsets {offsets}")
        q, k = workloads.generate_custom(shape, dtype, seed=seed + sum(shape))
        grid = tuple(n + o for n, o in zip(shape[1:4], offsets))
        want_q, want_k = oracle.rope3d_qk(q, k, dtype, split, 10000.0, offsets=offsets, grid=grid)
        dq, dk = to_dev(q, dtype), to_dev(k, dtype)
        for path in (0, 2):
            rla.set_option(rla.OPT_PATH, path)
            qo, ko = rla.forward_pair(dq, dk, split, 10000.0, grid=grid,
                                      offsets=None if offsets == (0, 0, 0) else offsets)
            torch.cuda.synchronize()
            assert_bitexact(to_host(qo, dtype), want_q, dtype, f"q {shape} {split} path {path}")
            assert_bitexact(to_host(ko, dtype), want_k, dtype, f"k {shape} {split} path {path}")
    assert rla.stats()["gate_disabled"] == 0


def test_misaligned_views_use_plain_kernel():
    shape, split = (1, 3, 4, 5, 4, 32), (8, 8, 16)
    q, k = workloads.generate_custom(shape, oracle.BF16, seed=5)
    n = q.size
    big = torch.empty(2 * n + 16, dtype=torch.bfloat16, device=DEV)
    dq = big[2:2 + n].view(shape)  # 4-byte aligned, not 16-byte aligned
    dk = big[n + 6:2 * n + 6].view(shape)
    dq.copy_(to_dev(q, oracle.BF16))
    dk.copy_(to_dev(k, oracle.BF16))
    with rla.tables_build(3, 4, 5, split) as tab:
        assert rla.kernel_choice(dq, dk, tab) == "plain"
        qo, ko = rla.apply_qk(dq, dk, tab)
    want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split)
    assert_bitexact(to_host(qo, oracle.BF16), want_q, oracle.BF16, "q")
    assert_bitexact(to_host(ko, oracle.BF16), want_k, oracle.BF16, "k")
    assert rla.stats()["plain_launches"] == 1


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.F32])
def test_special_values(dtype):
    """Tiny (subnormal-producing), huge, zero, signed-zero, infinite and NaN inputs."""
    shape, split = (1, 3, 4, 5, 2, 32), (8, 8, 16)
    rng = np.random.Generator(np.random.PCG64(77))
    vals = np.array([0.0, -0.0, 1e-38, -1e-38, 3e-39, 1e-40, 6e-45, 1e38, -3e38, 65504.0, np.inf, -np.inf, np.nan,
                     1.0, -1.0, 0.5], dtype=np.float32)
    x = vals[rng.integers(0, len(vals), size=2 * int(np.prod(shape)))].reshape((2,) + shape)
    if dtype == oracle.BF16:
        x = oracle.f32_to_bf16_bits(x)
    q, k = x[0], x[1]
    want_q, want_k = oracle.rope3d_qk(q, k, dtype, split)
    for path in (1, 2):
        qo, ko = run(to_dev(q, dtype), to_dev(k, dtype), split, path=path)
        assert_bitexact(to_host(qo, dtype), want_q, dtype, f"q path {path}")
        assert_bitexact(to_host(ko, dtype), want_k, dtype, f"k path {path}")


# ---------------------------------------------------------------------------
# full-size workloads: sampled tokens against the oracle, fast == plain in full
# ---------------------------------------------------------------------------

def full_check(x_host, out_dev, dtype, split, base, what):
    """Every element of out_dev against the oracle applied to x_host (raw bits)."""
    got = to_host(out_dev, dtype)
    n, first = oracle_full.compare_full(x_host, got, dtype, split, base)
    log(f"{what}: {x_host.size} elements compared with the oracle, {n} differ")
    assert n == 0, f"{what}: {n} of {x_host.size} elements differ from the oracle, first {first}"


def fast_equals_plain(dq, dk, qo, ko, split, base):
    rla.set_option(rla.OPT_PATH, 2)
    with rla.tables_build(*dq.shape[1:4], split, base) as tab:
        pq, pk = rla.apply_qk(dq, dk, tab)
    rla.set_option(rla.OPT_PATH, 0)
    torch.cuda.synchronize()
    assert torch.equal(qo.view(torch.int16), pq.view(torch.int16))
    assert torch.equal(ko.view(torch.int16), pk.view(torch.int16))


def test_workload3_24_calls_one_table_set():
    w = workloads.WORKLOADS[3]
    log("workload 3: generating inputs")
    (q, k), = workloads.generate(w)
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    outs = []
    for call in range(24):
        with rla.tables_build(*w.grids[0], w.split, w.base) as tab:
            outs.append(rla.apply_qk(dq, dk, tab))
    torch.cuda.synchronize()
    s = rla.stats()
    assert (s["cache_misses"], s["cache_hits"]) == (1, 23)
    assert s["gate_verifications"] == 1 and s["gate_trusted"] == 1 and s["fast_launches"] == 24
    q0, k0 = outs[0]
    for qo, ko in outs[1:]:
        assert torch.equal(qo.view(torch.int16), q0.view(torch.int16))
        assert torch.equal(ko.view(torch.int16), k0.view(torch.int16))
    full_check(q, q0, w.dtype, w.split, w.base, "workload 3 q")
    full_check(k, k0, w.dtype, w.split, w.base, "workload 3 k")
    fast_equals_plain(dq, dk, q0, k0, w.split, w.base)


def test_workload4_outliers():
    w = workloads.WORKLOADS[4]
    log("workload 4: generating inputs")
    (q, k), = workloads.generate(w)
    assert (oracle.to_f32(q[..., :64], w.dtype) == 60.0).any() and (oracle.to_f32(k[..., :64], w.dtype) == -60.0).any()
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    qo, ko = run(dq, dk, w.split, w.base)
    full_check(q, qo, w.dtype, w.split, w.base, "workload 4 q")
    full_check(k, ko, w.dtype, w.split, w.base, "workload 4 k")
    fast_equals_plain(dq, dk, qo, ko, w.split, w.base)


def test_fp32_at_workload4_size():
    """The fp32 fast kernel (two pairs per vector) at full size: workload 4's geometry in fp32
    (1.8 GB per tensor), every element against the oracle and fast == plain over the whole output."""
    shape, split = (1, 16, 96, 96, 24, 128), (32, 48, 48)
    log("fp32 at workload 4 size: generating inputs")
    q, k = workloads.generate_custom(shape, oracle.F32, seed=44)
    dq, dk = to_dev(q, oracle.F32), to_dev(k, oracle.F32)
    qo, ko = run(dq, dk, split)
    assert rla.stats()["fast_launches"] >= 1 and rla.stats()["gate_disabled"] == 0
    full_check(q, qo, oracle.F32, split, 10000.0, "fp32 at workload 4 size q")
    full_check(k, ko, oracle.F32, split, 10000.0, "fp32 at workload 4 size k")
    del q, k
    fast_equals_plain(dq, dk, qo, ko, split, 10000.0)


def test_workload5_three_alternating_grids():
    w = workloads.WORKLOADS[5]
    log("workload 5: generating inputs for three grids")
    data = workloads.generate(w)
    dev = [(to_dev(q, w.dtype), to_dev(k, w.dtype)) for q, k in data]
    results = {}
    for gi in w.calls:
        with rla.tables_build(*w.grids[gi], w.split, w.base) as tab:
            qo, ko = rla.apply_qk(dev[gi][0], dev[gi][1], tab)
        if gi in results:
            torch.cuda.synchronize()
            assert torch.equal(qo.view(torch.int16), results[gi][0].view(torch.int16))
            assert torch.equal(ko.view(torch.int16), results[gi][1].view(torch.int16))
        else:
            results[gi] = (qo, ko)
    torch.cuda.synchronize()
    s = rla.stats()
    assert (s["cache_misses"], s["cache_hits"], s["cache_evictions"]) == (3, 9, 0)
    assert s["gate_verifications"] == 3 and s["gate_trusted"] == 3
    for gi in range(3):
        full_check(data[gi][0], results[gi][0], w.dtype, w.split, w.base, f"workload 5 grid {gi} q")
        full_check(data[gi][1], results[gi][1], w.dtype, w.split, w.base, f"workload 5 grid {gi} k")
        fast_equals_plain(dev[gi][0], dev[gi][1], results[gi][0], results[gi][1], w.split, w.base)


def test_unit_vectors_full_size_workload5():
    """Pairs (1, 0) read back the bf16-rounded table row of every token, at the full size."""
    w = workloads.WORKLOADS[5]
    B, T, H, W, heads, D = w.shape(0)
    tabs = oracle.grid_tables(T, H, W, w.split, w.base)
    ct = np.concatenate([np.broadcast_to(tabs[0][0][:, None, None, :], (T, H, W, w.split[0] // 2)),
                         np.broadcast_to(tabs[1][0][None, :, None, :], (T, H, W, w.split[1] // 2)),
                         np.broadcast_to(tabs[2][0][None, None, :, :], (T, H, W, w.split[2] // 2))], axis=-1)
    st = np.concatenate([np.broadcast_to(tabs[0][1][:, None, None, :], (T, H, W, w.split[0] // 2)),
                         np.broadcast_to(tabs[1][1][None, :, None, :], (T, H, W, w.split[1] // 2)),
                         np.broadcast_to(tabs[2][1][None, None, :, :], (T, H, W, w.split[2] // 2))], axis=-1)
    exp_c = to_dev(oracle.f32_to_bf16_bits(ct), oracle.BF16)[None, :, :, :, None, :]
    exp_s = to_dev(oracle.f32_to_bf16_bits(st), oracle.BF16)[None, :, :, :, None, :]
    q = torch.zeros(w.shape(0), dtype=torch.bfloat16, device=DEV)
    q[..., 0::2] = 1.0
    k = torch.zeros_like(q)
    k[..., 1::2] = 1.0
    qo, ko = run(q, k, w.split, w.base)
    qv = qo.view(B, T, H, W, heads, D // 2, 2)
    kv = ko.view(B, T, H, W, heads, D // 2, 2)
    assert torch.equal(qv[..., 0].view(torch.int16), exp_c.expand(B, T, H, W, heads, D // 2).view(torch.int16))
    assert torch.equal(qv[..., 1].view(torch.int16), exp_s.expand(B, T, H, W, heads, D // 2).view(torch.int16))
    # (0, 1) -> (-sin, cos); compared by value: where sin is +0 the result is 0 - 0 = +0, not -0
    assert bool((kv[..., 0] == (-exp_s)).all())
    assert torch.equal(kv[..., 1].view(torch.int16), exp_c.expand(B, T, H, W, heads, D // 2).view(torch.int16))


# ---------------------------------------------------------------------------
# boundary behaviour: guard bands, gate, precheck on device pointers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", [1, 2], ids=["fast", "plain"])
def test_guard_bands_untouched(path):
    shape, split = (1, 3, 4, 5, 4, 32), (8, 8, 16)
    q, k = workloads.generate_custom(shape, oracle.BF16, seed=9)
    n = q.size
    guard = 4096
    buf = torch.full((2 * n + 3 * guard,), -7.0, dtype=torch.bfloat16, device=DEV)
    qo = buf[guard:guard + n].view(shape)
    ko = buf[2 * guard + n:2 * guard + 2 * n].view(shape)
    rla.set_option(rla.OPT_PATH, path)
    with rla.tables_build(3, 4, 5, split) as tab:
        rla.apply_qk(to_dev(q, oracle.BF16), to_dev(k, oracle.BF16), tab, qo, ko)
    torch.cuda.synchronize()
    for lo, hi in ((0, guard), (guard + n, 2 * guard + n), (2 * guard + 2 * n, buf.numel())):
        assert bool((buf[lo:hi] == -7.0).all()), (lo, hi)
    want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split)
    assert_bitexact(to_host(qo, oracle.BF16), want_q, oracle.BF16, "q")
    assert_bitexact(to_host(ko, oracle.BF16), want_k, oracle.BF16, "k")


def test_gate_forced_mismatch_falls_back_permanently():
    shape, split = (1, 2, 8, 8, 8, 64), (16, 24, 24)
    q, k = workloads.generate_custom(shape, oracle.BF16, seed=3)
    dq, dk = to_dev(q, oracle.BF16), to_dev(k, oracle.BF16)
    want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split)
    rla.set_option(rla.OPT_FORCE_GATE_MISMATCH, 1)
    with rla.tables_build(2, 8, 8, split) as tab:
        qo, ko = rla.apply_qk(dq, dk, tab)
        rla.set_option(rla.OPT_FORCE_GATE_MISMATCH, 0)
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "DISABLED"
        s = rla.stats()
        assert s["gate_verifications"] == 1 and s["gate_disabled"] == 1
        assert s["fast_launches"] == 1 and s["plain_launches"] == 1
        assert_bitexact(to_host(qo, oracle.BF16), want_q, oracle.BF16, "q after fallback")
        # later calls stay on the plain kernel, even with the forcing switched off
        for _ in range(3):
            qo, ko = rla.apply_qk(dq, dk, tab)
        torch.cuda.synchronize()
        s = rla.stats()
        assert s["plain_launches"] == 4 and s["fast_launches"] == 1 and s["gate_verifications"] == 1
        assert_bitexact(to_host(ko, oracle.BF16), want_k, oracle.BF16, "k on the plain path")
    # another configuration is unaffected
    shape2 = (2,) + shape[1:]
    q2, k2 = workloads.generate_custom(shape2, oracle.BF16, seed=4)
    with rla.tables_build(2, 8, 8, split) as tab:
        rla.apply_qk(to_dev(q2, oracle.BF16), to_dev(k2, oracle.BF16), tab)
    assert rla.gate_state(0, rla.DTYPE_BF16, shape2, split) == "TRUSTED"


def test_gate_trusted_then_no_more_verification():
    shape, split = (1, 2, 4, 4, 8, 64), (16, 24, 24)
    q, k = workloads.generate_custom(shape, oracle.BF16, seed=8)
    dq, dk = to_dev(q, oracle.BF16), to_dev(k, oracle.BF16)
    with rla.tables_build(2, 4, 4, split) as tab:
        for _ in range(5):
            rla.apply_qk(dq, dk, tab)
    torch.cuda.synchronize()
    s = rla.stats()
    assert s["gate_verifications"] == 1 and s["fast_launches"] == 5 and s["plain_launches"] == 0
    assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "TRUSTED"


def test_precheck_on_device_pointers():
    shape, split = (1, 2, 3, 4, 2, 12), (4, 4, 4)
    q = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros_like(q)
    with rla.tables_build(2, 3, 4, split) as tab:
        assert rla.can_use(q, k, tab) == (True, "OK")
        # host memory is refused
        hq = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
        L = _lib.lib()
        reason = ctypes.c_int(0)
        qo = torch.empty_like(q)
        ko = torch.empty_like(k)
        assert L.ltx3drope_can_use(qo.data_ptr(), ko.data_ptr(), hq.data_ptr(), k.data_ptr(), _lib.DTYPE_BF16, *shape,
                                   tab.handle, ctypes.byref(reason)) == 0
        assert _lib.REASONS[reason.value] == "NOT_DEVICE_PTR"
        # a device allocation too small for the claimed shape (the 2 MiB small-block segment of torch's
        # allocator cannot hold 115 MB); apply_qk is only called once can_use has refused, so nothing
        # can launch on the undersized buffer
        small = torch.empty(64, dtype=torch.bfloat16, device=DEV)
        big_shape = (1, 2, 3, 4, 200000, 12)
        assert L.ltx3drope_can_use(None, None, small.data_ptr(), small.data_ptr(), _lib.DTYPE_BF16, *big_shape,
                                   tab.handle, ctypes.byref(reason)) == 0
        assert _lib.REASONS[reason.value] == "EXTENT"
        st = L.ltx3drope_apply_qk(qo.data_ptr(), ko.data_ptr(), small.data_ptr(), small.data_ptr(),
                                  _lib.DTYPE_BF16, *big_shape, tab.handle, None)
        assert st == _lib.E_UNSUPPORTED
        # wrong grid for the tables -> table mismatch, nothing launched
        q2 = torch.zeros((1, 2, 3, 5, 2, 12), dtype=torch.bfloat16, device=DEV)
        with pytest.raises(rla.Ltx3dRopeUnsupported) as ei:
            rla.apply_qk(q2, q2.clone(), tab)
        assert ei.value.reason == "TABLE_GRID"
        # empty tensor, unsupported dtype, non-contiguous
        with pytest.raises(rla.Ltx3dRopeUnsupported):
            rla.apply_qk(q[:0], k[:0], tab)
        with pytest.raises(rla.Ltx3dRopeUnsupported):
            rla.apply_qk(q.half(), k.half(), tab)
        assert rla.can_use(q.transpose(1, 2), k.transpose(1, 2), tab)[0] is False
    assert rla.stats()["fast_launches"] == 0 and rla.stats()["plain_launches"] == 0


def test_host_table_mode_refuses_apply_and_names_it():
    """Tables built in host-table test mode pass the precheck (its memory checks are skipped), but no
    apply entry point launches with them; the binding names that refusal HOST_MODE."""
    shape, split = (1, 2, 3, 4, 2, 12), (4, 4, 4)
    q = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros_like(q)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    rla.set_option(rla.OPT_HOST_TABLES, 1)
    try:
        with rla.tables_build(2, 3, 4, split) as tab:
            assert rla.can_use(q, k, tab) == (True, "OK")
            for call in (lambda: rla.apply_qk(q, k, tab), lambda: rla.apply_qk_noalloc(q, k, tab, qo, ko)):
                with pytest.raises(rla.Ltx3dRopeUnsupported) as ei:
                    call()
                assert ei.value.reason == "HOST_MODE" and ei.value.status == _lib.E_UNSUPPORTED
    finally:
        rla.set_option(rla.OPT_HOST_TABLES, 0)
        rla.cache_clear()
    s = rla.stats()
    assert s["fast_launches"] == 0 and s["plain_launches"] == 0 and s["rejected"] == 2


def test_side_stream_and_forward_pair():
    shape, split = (1, 4, 8, 8, 16, 128), (32, 48, 48)
    q, k = workloads.generate_custom(shape, oracle.BF16, seed=12)
    want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split)
    s = torch.cuda.Stream()
    dq, dk = to_dev(q, oracle.BF16), to_dev(k, oracle.BF16)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        qo, ko = rla.forward_pair(dq, dk, split)
    s.synchronize()
    assert_bitexact(to_host(qo, oracle.BF16), want_q, oracle.BF16, "q")
    assert_bitexact(to_host(ko, oracle.BF16), want_k, oracle.BF16, "k")


def test_concurrent_first_calls_from_threads():
    """First calls of four new configurations started together from host threads, each on its own
    stream: the gate's verifications share one device counter and must not disturb each other."""
    import threading
    cases = [((1, 2, 4, 4, 8, 64), (16, 24, 24)), ((1, 3, 4, 6, 4, 96), (32, 32, 32)),
             ((2, 2, 3, 5, 6, 64), (16, 16, 32)), ((1, 4, 2, 8, 8, 128), (32, 48, 48))]
    inputs = [workloads.generate_custom(shape, oracle.BF16, seed=30 + i) for i, (shape, _) in enumerate(cases)]
    dev_in = [(to_dev(q, oracle.BF16), to_dev(k, oracle.BF16)) for q, k in inputs]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    results, errors = [None] * len(cases), []
    start = threading.Barrier(len(cases))

    def worker(i):
        try:
            start.wait(timeout=60)
            with torch.cuda.stream(streams[i]):
                results[i] = rla.forward_pair(*dev_in[i], cases[i][1])
            streams[i].synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i, (shape, split) in enumerate(cases):
        want_q, want_k = oracle.rope3d_qk(*inputs[i], oracle.BF16, split)
        assert_bitexact(to_host(results[i][0], oracle.BF16), want_q, oracle.BF16, f"q{i}")
        assert_bitexact(to_host(results[i][1], oracle.BF16), want_k, oracle.BF16, f"k{i}")
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "TRUSTED"
    s = rla.stats()
    assert s["gate_verifications"] == len(cases) and s["gate_disabled"] == 0


def test_copy_helper():
    src = torch.randint(-1000, 1000, (1 << 20,), dtype=torch.int32, device=DEV)
    dst = torch.empty_like(src)
    rla.copy_bytes(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# ---------------------------------------------------------------------------
# shards of a larger grid and in-place mode
# ---------------------------------------------------------------------------

SHARDS = [
    # full grid (T, H, W), local shape, offsets, split, dtype
    ((9, 6, 7), (2, 3, 6, 7, 4, 32), (5, 0, 0), (8, 8, 16), oracle.BF16),
    ((4, 10, 7), (1, 4, 3, 7, 3, 24), (0, 6, 0), (8, 8, 8), oracle.BF16),
    ((4, 5, 12), (1, 4, 5, 5, 2, 48), (0, 0, 7), (16, 16, 16), oracle.F32),
    ((6, 8, 9), (2, 2, 3, 4, 8, 64), (3, 2, 5), (16, 24, 24), oracle.BF16),
    ((6, 8, 9), (1, 2, 3, 4, 3, 12), (1, 4, 2), (2, 6, 4), oracle.BF16),  # plain kernel only
    ((6, 8, 9), (1, 2, 3, 4, 16, 96), (2, 3, 4), (30, 34, 32), oracle.BF16),  # LDS-assembled table row
]


@pytest.mark.parametrize("grid,shape,offsets,split,dtype", SHARDS, ids=[str(s[2]) + s[4] for s in SHARDS])
@pytest.mark.parametrize("path", [0, 2], ids=["auto", "plain"])
def test_shards_full(grid, shape, offsets, split, dtype, path):
    log(f"shard {shape} at {offsets} of {grid}, path {path}")
    q, k = workloads.generate_custom(shape, dtype, seed=sum(offsets) + 100)
    want_q, want_k = oracle.rope3d_qk(q, k, dtype, split, offsets=offsets, grid=grid)
    rla.set_option(rla.OPT_PATH, path)
    with rla.tables_build(*grid, split) as tab:
        qo, ko = rla.apply_qk(to_dev(q, dtype), to_dev(k, dtype), tab, offsets=offsets)
    torch.cuda.synchronize()
    assert_bitexact(to_host(qo, dtype), want_q, dtype, "q")
    assert_bitexact(to_host(ko, dtype), want_k, dtype, "k")


def test_frame_shards_of_workload4_match_the_full_result():
    """Sequence parallelism over frames at full size: workload 4 split into 8 frame shards
    (2 frames each, t_offset = 2r) with the whole grid's tables; every shard's output equals
    the same slab of the unsharded output, which is itself checked against the oracle."""
    w = workloads.WORKLOADS[4]
    log("workload 4 frame shards: generating inputs")
    (q, k), = workloads.generate(w)
    dq, dk = to_dev(q, w.dtype), to_dev(k, w.dtype)
    with rla.tables_build(*w.grids[0], w.split, w.base) as tab:
        fq, fk = rla.apply_qk(dq, dk, tab)
        T = w.grids[0][0]
        per = T // 8
        for r in range(8):
            sl = slice(r * per, (r + 1) * per)
            sq, sk = dq[:, sl].contiguous(), dk[:, sl].contiguous()
            oq, ok = rla.apply_qk(sq, sk, tab, offsets=(r * per, 0, 0))
            assert torch.equal(oq.view(torch.int16), fq[:, sl].view(torch.int16)), r
            assert torch.equal(ok.view(torch.int16), fk[:, sl].view(torch.int16)), r
    torch.cuda.synchronize()
    full_check(q, fq, w.dtype, w.split, w.base, "workload 4 (unsharded reference of the shards) q")
    full_check(k, fk, w.dtype, w.split, w.base, "workload 4 (unsharded reference of the shards) k")
    # a spatial tile as well: rows 32..63, columns 64..95 of every frame
    with rla.tables_build(*w.grids[0], w.split, w.base) as tab:
        tq = dq[:, :, 32:64, 64:96].contiguous()
        tk = dk[:, :, 32:64, 64:96].contiguous()
        oq, ok = rla.apply_qk(tq, tk, tab, offsets=(0, 32, 64))
    torch.cuda.synchronize()
    assert torch.equal(oq.view(torch.int16), fq[:, :, 32:64, 64:96].view(torch.int16))
    assert torch.equal(ok.view(torch.int16), fk[:, :, 32:64, 64:96].view(torch.int16))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.F32])
def test_inplace_matches_out_of_place_and_respects_the_gate(dtype):
    shape, split = (1, 3, 8, 8, 8, 64), (16, 24, 24)
    q, k = workloads.generate_custom(shape, dtype, seed=31)
    want_q, want_k = oracle.rope3d_qk(q, k, dtype, split)
    with rla.tables_build(3, 8, 8, split) as tab:
        # unseen configuration: an in-place call cannot be verified, so it runs the plain kernel
        dq, dk = to_dev(q, dtype), to_dev(k, dtype)
        rq, rk = rla.apply_qk(dq, dk, tab, inplace=True)
        torch.cuda.synchronize()
        assert rq.data_ptr() == dq.data_ptr() and rk.data_ptr() == dk.data_ptr()
        s = rla.stats()
        assert s["plain_launches"] == 1 and s["fast_launches"] == 0 and s["gate_verifications"] == 0
        assert rla.gate_state(0, rla.DTYPE_BF16 if dtype == oracle.BF16 else rla.DTYPE_F32, shape, split) == "UNSEEN"
        assert_bitexact(to_host(dq, dtype), want_q, dtype, "q in place (plain)")
        assert_bitexact(to_host(dk, dtype), want_k, dtype, "k in place (plain)")
        # an out-of-place call verifies and trusts the fast kernel; later in-place calls use it
        rla.apply_qk(to_dev(q, dtype), to_dev(k, dtype), tab)
        dq, dk = to_dev(q, dtype), to_dev(k, dtype)
        rla.apply_qk(dq, dk, tab, inplace=True)
        torch.cuda.synchronize()
        s = rla.stats()
        assert s["gate_verifications"] == 1 and s["fast_launches"] == 2
        assert_bitexact(to_host(dq, dtype), want_q, dtype, "q in place (fast)")
        assert_bitexact(to_host(dk, dtype), want_k, dtype, "k in place (fast)")


def test_largest_supported_tensor():
    """31 heads x [1, 16, 64, 1024] x head_dim 128 = 4,160,749,568 elements per tensor (7.75 GiB of
    bf16), just under the 2^32 limit: the gate's full-size verification, fast == plain over the
    whole output, and every element of Q and K against the oracle; one more head (2^32 elements)
    is refused without a launch.  Inputs are finite random bf16 patterns drawn on the device."""
    shape, split = (1, 16, 64, 1024, 31, 128), (32, 48, 48)
    log("largest tensor: generating inputs on the device")
    dq = workloads.generate_bf16_bits(shape, 101, DEV)
    dk = workloads.generate_bf16_bits(shape, 102, DEV)
    with rla.tables_build(16, 64, 1024, split) as tab:
        too_big = (1, 16, 64, 1024, 32, 128)
        reason = ctypes.c_int(0)
        assert _lib.lib().ltx3drope_can_use(None, None, dq.data_ptr(), dk.data_ptr(), _lib.DTYPE_BF16, *too_big,
                                            tab.handle, ctypes.byref(reason)) == 0
        assert _lib.REASONS[reason.value] == "TOO_LARGE"
        qo, ko = rla.apply_qk(dq, dk, tab)  # first call: fast kernel verified against the plain one
        torch.cuda.synchronize()
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "TRUSTED"
        rla.set_option(rla.OPT_PATH, 2)
        pq, pk = rla.apply_qk(dq, dk, tab)
        torch.cuda.synchronize()
        assert torch.equal(qo.view(torch.int16), pq.view(torch.int16))
        assert torch.equal(ko.view(torch.int16), pk.view(torch.int16))
        del pq, pk
    log("largest tensor: oracle comparison of every element")
    for x, out, name in ((dq, qo, "q"), (dk, ko, "k")):
        full_check(to_host(x, oracle.BF16), out, oracle.BF16, split, 10000.0, f"largest tensor {name}")


def test_tensor_above_2_to_the_32_elements_runs_in_batch_slices():
    """B = 2 batch elements of [16, 64, 1024] x 17 heads x head_dim 128 = 2,281,701,376 elements
    each: 4,563,402,752 elements per tensor (8.5 GiB of bf16), above 2^32, so each kernel runs as
    two launches of one batch element.  The gate verifies both slices, fast == plain over the
    whole output, and every element of Q_out and K_out is compared with the oracle."""
    shape, split = (2, 16, 64, 1024, 17, 128), (32, 48, 48)
    log("above 2^32 elements: generating inputs on the device")
    dq = workloads.generate_bf16_bits(shape, 201, DEV)
    dk = workloads.generate_bf16_bits(shape, 202, DEV)
    with rla.tables_build(16, 64, 1024, split) as tab:
        assert rla.can_use(dq, dk, tab) == (True, "OK")
        qo, ko = rla.apply_qk(dq, dk, tab)
        torch.cuda.synchronize()
        s = rla.stats()
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "TRUSTED"
        assert s["gate_verifications"] == 1 and s["fast_launches"] == 2 and s["plain_launches"] == 0
        rla.set_option(rla.OPT_PATH, 2)
        pq, pk = rla.apply_qk(dq, dk, tab)
        torch.cuda.synchronize()
        assert rla.stats()["plain_launches"] == 2
        assert torch.equal(qo.view(torch.int16), pq.view(torch.int16))
        assert torch.equal(ko.view(torch.int16), pk.view(torch.int16))
        del pq, pk
    log("above 2^32 elements: oracle comparison of every element")
    for x, out, name in ((dq, qo, "q"), (dk, ko, "k")):
        full_check(to_host(x, oracle.BF16), out, oracle.BF16, split, 10000.0, f"above 2^32 elements {name}")


def test_each_shard_placement_is_verified_on_its_first_call():
    """The gate's key holds the tables' grid and the shard's offsets: a slab of a larger grid is
    verified on its own first call, a repeated placement is not verified again, and every
    output equals the oracle."""
    grid, shape, split = (6, 8, 9), (1, 2, 3, 4, 8, 64), (16, 24, 24)
    q, k = workloads.generate_custom(shape, oracle.BF16, seed=77)
    dq, dk = to_dev(q, oracle.BF16), to_dev(k, oracle.BF16)
    placements = [(0, 0, 0), (3, 2, 5), (3, 2, 5), (1, 4, 2)]
    with rla.tables_build(*grid, split) as tab:
        for offsets in placements:
            qo, ko = rla.apply_qk(dq, dk, tab, offsets=offsets)
            torch.cuda.synchronize()
            want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split, offsets=offsets, grid=grid)
            assert_bitexact(to_host(qo, oracle.BF16), want_q, oracle.BF16, f"q at {offsets}")
            assert_bitexact(to_host(ko, oracle.BF16), want_k, oracle.BF16, f"k at {offsets}")
    s = rla.stats()
    assert s["gate_verifications"] == 3 and s["gate_trusted"] == 3 and s["fast_launches"] == 4
