"""Property test of the 3D RoPE precheck (ltx3drope_can_use and ltx3drope_can_use_shard) against a
model of its documented rule list, on the CPU.

The model below restates the rules of include/ltx3drope.h in their documented order (the first
failing rule names the reason): null pointers, dtype, positive sizes, the split sum, the grid rule
(exact grid, or the shard's containment), pair alignment, the size limits, then overlaps (exact
in-place aliasing allowed with a shard's in-place flag).  Hypothesis draws shapes, splits, table
grids, shard descriptors and pointer layouts around each rule's boundary; every draw must give the
library's verdict.  Tables are built in host-table mode, so no pointer is dereferenced and nothing
touches HIP (the device-memory rules come last and are skipped in that mode).
"""
from __future__ import annotations

import ctypes
import os

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libltx3drope.so not built (python -m rope_ltx3drope_amd.build)", allow_module_level=True)

L = _lib.lib()
BASE = 1 << 56  # fake addresses: never dereferenced in host-table mode


@pytest.fixture(scope="module", autouse=True)
def host_mode():
    rla.set_option(rla.OPT_HOST_TABLES, 1)
    rla.cache_clear()
    yield
    rla.cache_clear()
    rla.set_option(rla.OPT_HOST_TABLES, 0)


def model(api, ptrs, dtype, dims, split, tab_grid, shard):
    """The documented verdict (a reason name)."""
    q_out, k_out, q, k = ptrs
    B, T, H, W, heads, D = dims
    if api == "shard" and shard is not None:
        t0, h0, w0, inplace, reserved = shard
        if reserved != 0 or inplace not in (0, 1) or min(t0, h0, w0) < 0:
            return "TABLE_GRID"
    outputs = q_out is not None or k_out is not None
    if (outputs and (q_out is None or k_out is None)) or q is None or k is None:
        return "NULLPTR"
    if dtype not in (_lib.DTYPE_F32, _lib.DTYPE_BF16):
        return "DTYPE"
    if min(dims) <= 0:
        return "NONPOSITIVE_DIM"
    if D != sum(split):
        return "SPLIT_SUM"
    if api == "plain":
        if (T, H, W) != tab_grid:
            return "TABLE_GRID"
        offsets, inplace = (0, 0, 0), 0
    else:
        offsets, inplace = ((0, 0, 0), 0) if shard is None else (shard[:3], shard[3])
        if any(o + n > g for o, n, g in zip(offsets, (T, H, W), tab_grid)):
            return "TABLE_GRID"
    es = 4 if dtype == _lib.DTYPE_F32 else 2
    for p in ((q, k, q_out, k_out) if outputs else (q, k)):
        if p % (2 * es):
            return "ALIGN"
    per_batch = T * H * W * heads * D
    if max(T, H, W, heads, D, B) >= 1 << 31 or per_batch >= 1 << 32 or B * per_batch > 1 << 48:
        return "TOO_LARGE"
    if outputs:
        n = B * per_batch * es

        def overlap(a, b):
            return a < b + n and b < a + n

        q_ok = inplace == 1 and q_out == q
        k_ok = inplace == 1 and k_out == k
        if ((not q_ok and overlap(q_out, q)) or overlap(q_out, k) or overlap(k_out, q)
                or (not k_ok and overlap(k_out, k)) or overlap(q_out, k_out)):
            return "OVERLAP"
    return "OK"


SPLITS = [(2, 2, 2), (4, 4, 4), (8, 4, 2), (4, 4, 8), (32, 48, 48), (6, 10, 14)]
BIG = [1 << 20, (1 << 31) - 1, 1 << 31, 1 << 32]


def usually(good, rare):
    """Mostly a valid value (so that draws reach the later rules), sometimes one at or past a
    rule's boundary."""
    return st.integers(0, 9).flatmap(lambda r: good if r < 8 else rare)


def size(good):
    """A size near a rule's boundary: a neighbour of the good value, zero, negative or huge."""
    return st.one_of(st.sampled_from([good - 1, good + 1, 0, -1]), st.sampled_from(BIG))


@st.composite
def size_limits(draw):
    """One token of head_dim 16 with head counts and batch sizes at the size limits: 2^32 elements
    per batch element (refused) and 2^48 in all (accepted; one more batch element is refused)."""
    heads = draw(st.sampled_from([(1 << 28) - 1, 1 << 28, 1 << 27]))
    B = draw(st.sampled_from([1, 1 << 17, (1 << 17) + 1, 1 << 16]))
    return B, heads


@st.composite
def cases(draw):
    api = draw(st.sampled_from(["plain", "shard"]))
    if draw(st.integers(0, 4)) == 0:
        split, tab_grid, local, D = (4, 4, 8), (1, 1, 1), (1, 1, 1), 16
        B, heads = draw(size_limits())
    else:
        split = draw(st.sampled_from(SPLITS))
        tab_grid = tuple(draw(st.integers(1, 6)) for _ in range(3))
        if api == "plain":
            local = tuple(draw(usually(st.just(g), size(g))) for g in tab_grid)
        else:
            local = tuple(draw(usually(st.integers(1, g), size(g))) for g in tab_grid)
        B = draw(usually(st.integers(1, 3), st.sampled_from([0, -1, 1 << 16, (1 << 31) - 1, 1 << 31])))
        heads = draw(usually(st.integers(1, 8), st.sampled_from([0, -1] + BIG)))
        D = draw(usually(st.just(sum(split)), size(sum(split))))
    dtype = draw(usually(st.sampled_from([_lib.DTYPE_F32, _lib.DTYPE_BF16]), st.sampled_from([2, -1])))
    shard = None
    if api == "shard" and draw(st.booleans()):
        shard = (draw(usually(st.integers(0, 3), st.just(-1))), draw(usually(st.integers(0, 3), st.just(-1))),
                 draw(usually(st.integers(0, 3), st.just(-1))), draw(usually(st.sampled_from([0, 1]), st.just(2))),
                 draw(usually(st.just(0), st.just(1))))
    # pointers: Q and K in their own regions, or aliasing; outputs absent, fresh, in place or near
    stride = 1 << 52  # far apart: fresh regions never overlap whatever the size
    q = BASE + draw(usually(st.sampled_from([0, 8, 16]), st.sampled_from([2, 4])))
    k = draw(st.sampled_from([BASE + stride, BASE + stride, q, q + 8, BASE + stride + 2]))
    kind = draw(st.sampled_from(["none", "fresh", "fresh", "fresh", "inplace", "inplace", "near", "one_null",
                                 "crossed", "null_q", "outputs_overlap", "q_out_on_k", "k_out_on_q", "k_out_near_k",
                                 "k_in_place_only", "touching"]))
    q_out = k_out = None
    if kind == "fresh":
        q_out, k_out = BASE + 2 * stride + draw(st.sampled_from([0, 8, 4])), BASE + 3 * stride
    elif kind == "inplace":
        q_out, k_out = q, draw(st.sampled_from([k, BASE + 3 * stride]))
    elif kind == "near":
        q_out, k_out = q + draw(st.sampled_from([-16, 16, 1 << 12])), BASE + 3 * stride
    elif kind == "one_null":
        q_out = BASE + 2 * stride
    elif kind == "crossed":
        q_out, k_out = k, q
    elif kind == "null_q":
        q = None
    elif kind == "q_out_on_k":
        q_out, k_out = k + draw(st.sampled_from([0, 16])), BASE + 3 * stride
    elif kind == "k_out_on_q":
        q_out, k_out = BASE + 2 * stride, q + draw(st.sampled_from([0, 16]))
    elif kind == "k_out_near_k":
        q_out, k_out = BASE + 2 * stride, k + draw(st.sampled_from([-16, 16]))
    elif kind == "k_in_place_only":
        q_out, k_out = BASE + 2 * stride, k
    elif kind == "touching":
        # Q_out ends exactly where Q starts (no overlap), or 8 bytes later (an overlap)
        B_, T_, H_, W_, h_, D_ = B, *local, heads, D
        n = B_ * T_ * H_ * W_ * h_ * D_ * (4 if dtype == _lib.DTYPE_F32 else 2) if min(B_, T_, H_, W_, h_, D_) > 0 else 16
        q_out, k_out = q - n + draw(st.sampled_from([0, 8])), BASE + 3 * stride
    elif kind == "outputs_overlap":
        q_out = BASE + 2 * stride
        k_out = q_out + draw(st.sampled_from([0, 16, 1 << 12]))
    return api, (q_out, k_out, q, k), dtype, (B, *local, heads, D), split, tab_grid, shard


_tables = {}


def tables(tab_grid, split):
    key = (tab_grid, split)
    if key not in _tables:
        _tables[key] = rla.tables_build(*tab_grid, split)
    return _tables[key]


def library(api, ptrs, dtype, dims, split, tab_grid, shard):
    tab = tables(tab_grid, split)
    reason = ctypes.c_int(-1)
    if api == "plain":
        ok = L.ltx3drope_can_use(*ptrs, dtype, *dims, tab.handle, ctypes.byref(reason))
    else:
        desc = None if shard is None else ctypes.byref(_lib.Shard(*shard))
        ok = L.ltx3drope_can_use_shard(*ptrs, dtype, *dims, desc, tab.handle, ctypes.byref(reason))
    return ok, _lib.REASONS[reason.value]


@settings(max_examples=1500, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(cases())
def test_precheck_matches_its_documented_rules(case):
    ok, got = library(*case)
    want = model(*case)
    assert got == want, (case, got, want)
    assert ok == (1 if want == "OK" else 0)


def test_model_reaches_every_reason():
    """The strategy reaches every rule (guards against a model that agrees only vacuously)."""
    seen = set()

    @settings(max_examples=1500, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
    @given(cases())
    def collect(case):
        seen.add(model(*case))

    collect()
    assert seen >= {"OK", "NULLPTR", "DTYPE", "NONPOSITIVE_DIM", "SPLIT_SUM", "TABLE_GRID", "ALIGN", "TOO_LARGE",
                    "OVERLAP"}, seen
