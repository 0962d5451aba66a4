"""CPU tests of the C-ABI library: exports, host-side table build, FIFO cache,
precheck rules, options and the gate state machine's host bookkeeping.

The library is loaded for real (it links the HIP runtime, which loads without
a GPU); the table cache runs in host-table mode, in which nothing calls HIP and
apply_qk refuses, so every test here is pure host logic.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import threading

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ltx3drope.h")

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libltx3drope.so not built (python -m rope_ltx3drope_amd.build)", allow_module_level=True)

L = _lib.lib()


@pytest.fixture(autouse=True)
def host_mode():
    rla.set_option(rla.OPT_HOST_TABLES, 1)
    rla.cache_clear()
    rla.stats_reset()
    yield
    rla.cache_clear()
    rla.set_option(rla.OPT_HOST_TABLES, 0)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ltx3drope_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_exactly_the_binding_exports():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True)
    syms = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
    for name in header_functions():
        assert name in syms, name
        assert getattr(L, name) is not None


def test_version_and_strings():
    assert rla.version() == 1
    assert _lib.status_string(0) == "ok"
    assert "precheck" in _lib.status_string(_lib.E_UNSUPPORTED)
    for code in _lib.REASONS:
        assert _lib.reason_string(code) != "unknown reason"


# ---------------------------------------------------------------------------
# tables: the library's host build equals the oracle's tables bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wk", [1, 2, 3, 4, 5])
def test_tables_equal_oracle_bitwise(wk):
    w = workloads.WORKLOADS[wk]
    for (T, H, W) in w.grids:
        with rla.tables_build(T, H, W, w.split, w.base) as tab:
            got = tab.read()
            assert tab.describe()["packed_pairs"] == T * w.split[0] // 2 + H * w.split[1] // 2 + W * w.split[2] // 2
        want = oracle.grid_tables(T, H, W, w.split, w.base)
        for (gc, gs), (wc, ws) in zip(got, want):
            np.testing.assert_array_equal(gc.view(np.uint32), wc.view(np.uint32))
            np.testing.assert_array_equal(gs.view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("grid,split,base", [((7, 3, 5), (2, 6, 10), 10000.0), ((1, 1, 1), (2, 2, 2), 500.0),
                                             ((300, 2, 9), (64, 4, 30), 1e6)])
def test_tables_equal_oracle_other_shapes(grid, split, base):
    with rla.tables_build(*grid, split, base) as tab:
        got = tab.read()
    want = oracle.grid_tables(*grid, split, base)
    for (gc, gs), (wc, ws) in zip(got, want):
        np.testing.assert_array_equal(gc.view(np.uint32), wc.view(np.uint32))
        np.testing.assert_array_equal(gs.view(np.uint32), ws.view(np.uint32))


def test_packed_layout():
    tab = rla.tables_build(2, 3, 4, (4, 6, 8), 10000.0)
    d = tab.describe()
    assert d["packed_pairs"] == 2 * 2 + 3 * 3 + 4 * 4
    packed = np.ctypeslib.as_array(ctypes.cast(d["packed"], ctypes.POINTER(ctypes.c_float)),
                                   shape=(2 * d["packed_pairs"],)).copy()
    (ct, st), (ch, sh), (cw, sw) = oracle.grid_tables(2, 3, 4, (4, 6, 8), 10000.0)
    want = np.concatenate([np.stack([c.reshape(-1), s.reshape(-1)], -1).reshape(-1)
                           for c, s in ((ct, st), (ch, sh), (cw, sw))])
    np.testing.assert_array_equal(packed.view(np.uint32), want.view(np.uint32))
    tab.close()


@pytest.mark.parametrize("args", [
    (0, 0, 4, 4, 2, 2, 2, 1e4), (0, 4, -1, 4, 2, 2, 2, 1e4), (0, 4, 4, 4, 3, 2, 2, 1e4), (0, 4, 4, 4, 2, 0, 2, 1e4),
    (0, 4, 4, 4, 2, 2, 2, 0.0), (0, 4, 4, 4, 2, 2, 2, float("inf")), (0, 4, 4, 4, 2, 2, 2, float("nan")),
    (-1, 4, 4, 4, 2, 2, 2, 1e4), (0, 1 << 40, 4, 4, 2, 2, 2, 1e4),
])
def test_tables_build_rejects_bad_arguments(args):
    out = ctypes.c_void_p()
    assert L.ltx3drope_tables_build(*args, None, ctypes.byref(out)) == _lib.E_INVALID
    assert not out.value
    assert L.ltx3drope_tables_build(0, 2, 2, 2, 2, 2, 2, 1e4, None, None) == _lib.E_INVALID


# ---------------------------------------------------------------------------
# FIFO cache ("Implementation breakdown", step 1: at most 16 entries, FIFO)
# ---------------------------------------------------------------------------

def test_cache_hit_returns_same_tables_and_counts():
    a = rla.tables_build(8, 64, 64, (32, 48, 48))
    for _ in range(23):  # the other 23 decoder blocks on the same grid
        b = rla.tables_build(8, 64, 64, (32, 48, 48))
        assert b.describe()["packed"] == a.describe()["packed"]
        b.close()
    s = rla.stats()
    assert (s["cache_misses"], s["cache_hits"], s["cache_live"]) == (1, 23, 1)
    a.close()


def test_cache_key_includes_split_base_and_device():
    base = rla.tables_build(4, 4, 4, (2, 2, 4), 10000.0)
    others = [rla.tables_build(4, 4, 4, (4, 2, 2), 10000.0), rla.tables_build(4, 4, 4, (2, 2, 4), 500.0),
              rla.tables_build(4, 4, 4, (2, 2, 4), 10000.0, device=1), rla.tables_build(4, 4, 5, (2, 2, 4), 10000.0)]
    ptrs = {t.describe()["packed"] for t in [base] + others}
    assert len(ptrs) == 5
    assert rla.stats()["cache_misses"] == 5


def test_cache_fifo_eviction_and_no_lru_refresh():
    grids = [(1, 1, g + 1) for g in range(17)]
    held = rla.tables_build(*grids[0], (2, 2, 2))
    first_ptr = held.describe()["packed"]
    for g in grids[1:16]:
        rla.tables_build(*g, (2, 2, 2)).close()
    # a hit on the oldest entry must not refresh it (FIFO, not LRU)
    rla.tables_build(*grids[0], (2, 2, 2)).close()
    s = rla.stats()
    assert (s["cache_live"], s["cache_evictions"], s["cache_hits"]) == (16, 0, 1)
    rla.tables_build(*grids[16], (2, 2, 2)).close()  # 17th grid evicts the oldest: grids[0]
    s = rla.stats()
    assert (s["cache_live"], s["cache_evictions"]) == (16, 1)
    # the caller's handle survives eviction
    assert held.describe()["packed"] == first_ptr
    before = held.read()
    # grids[1] is still cached; grids[0] was evicted and is rebuilt bit-identically
    misses = s["cache_misses"]
    rla.tables_build(*grids[1], (2, 2, 2)).close()
    assert rla.stats()["cache_misses"] == misses
    again = rla.tables_build(*grids[0], (2, 2, 2))
    assert rla.stats()["cache_misses"] == misses + 1
    assert again.describe()["packed"] != first_ptr
    for (a, b), (c, d) in zip(before, again.read()):
        np.testing.assert_array_equal(a.view(np.uint32), c.view(np.uint32))
        np.testing.assert_array_equal(b.view(np.uint32), d.view(np.uint32))
    again.close()
    held.close()


def test_alternating_grids_hit_after_first_pass():
    w = workloads.WORKLOADS[5]
    for gi in w.calls:
        rla.tables_build(*w.grids[gi], w.split, w.base).close()
    s = rla.stats()
    assert (s["cache_misses"], s["cache_hits"], s["cache_evictions"]) == (3, 9, 0)


def test_refcount_frees_when_last_reference_goes():
    rla.cache_clear()
    alive0 = rla.stats()["tables_alive"]
    t = rla.tables_build(3, 3, 3, (2, 2, 2))
    assert rla.stats()["tables_alive"] == alive0 + 1
    rla.cache_clear()  # cache drops its reference; ours keeps the object alive
    assert rla.stats()["tables_alive"] == alive0 + 1
    t.read()
    t.close()
    assert rla.stats()["tables_alive"] == alive0
    assert L.ltx3drope_tables_release(None) == _lib.E_INVALID
    # a closed handle refuses further use instead of touching freed memory; closing twice is harmless
    with pytest.raises(ValueError):
        t.describe()
    t.close()
    with rla.tables_build(3, 3, 3, (2, 2, 2)) as t2:
        assert t2.grid == (3, 3, 3) and t2.split == (2, 2, 2)
    with pytest.raises(ValueError):
        t2.read()


def test_concurrent_builds_are_consistent():
    errors = []

    def worker(i):
        try:
            for r in range(50):
                g = (1 + (i + r) % 5, 2, 3)
                t = rla.tables_build(*g, (2, 4, 2))
                assert t.grid == g
                t.close()
        except Exception as e:  # pragma: no cover
            errors.append(e)

    th = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors
    s = rla.stats()
    assert s["cache_live"] == 5
    assert s["cache_hits"] + s["cache_misses"] == 400


# ---------------------------------------------------------------------------
# precheck (golden rule list from the page)
# ---------------------------------------------------------------------------

def golden_rules():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "precheck_rules.txt")):
        if line.startswith("#") or not line.strip():
            continue
        rid, origin, reason, words = line.rstrip("\n").split("\t")
        rows.append((rid, origin, reason, words))
    return rows


SHAPE = (1, 2, 3, 4, 2, 12)
SPLIT = (4, 4, 4)
NUMEL = int(np.prod(SHAPE))


def call_can_use(q_out, k_out, q, k, dtype, shape, tab):
    reason = ctypes.c_int(-1)
    ok = L.ltx3drope_can_use(q_out, k_out, q, k, dtype, *shape, tab, ctypes.byref(reason))
    return ok, _lib.REASONS[reason.value]


def fake_ptrs(es, gap=1 << 20):
    base = 1 << 32
    return base, base + gap, base + 2 * gap, base + 3 * gap  # q, k, q_out, k_out


def case_for(rule, tab, tab_other_grid, tab_bad_split):
    """(args to can_use) violating exactly one rule, or None when the binding checks it."""
    es = 2
    q, k, qo, ko = fake_ptrs(es)
    d = _lib.DTYPE_BF16
    shp = SHAPE
    if rule == "dtype":
        return (qo, ko, q, k, 7, shp, tab)
    if rule == "positive_sizes":
        return (qo, ko, q, k, d, (1, 2, 3, 4, 0, 12), tab)
    if rule == "split_sum":
        return (qo, ko, q, k, d, (1, 2, 3, 4, 2, 14), tab)
    if rule == "table_grid":
        return (qo, ko, q, k, d, shp, tab_other_grid)
    if rule == "pair_alignment":
        return (qo, ko, q + 2, k, d, shp, tab)
    if rule == "null":
        return (qo, ko, None, k, d, shp, tab)
    if rule == "overlap":
        return (q + 64, ko, q, k, d, shp, tab)
    if rule == "too_large":
        return (qo, ko, q, k, d, (1, 1, 1, 1 << 10, 1 << 22, 12), None)
    return None


def test_precheck_rules_from_golden_list():
    tab = rla.tables_build(2, 3, 4, SPLIT)
    other = rla.tables_build(2, 3, 5, SPLIT)
    big = rla.tables_build(1, 1, 1 << 10, SPLIT)
    checked = 0
    for rid, origin, reason, _ in golden_rules():
        if rid == "split_even":
            # the split lives in the tables, which refuse an odd or empty chunk at build time
            out = ctypes.c_void_p()
            for bad in ((3, 4, 5), (0, 6, 6), (4, -2, 10)):
                assert L.ltx3drope_tables_build(0, 2, 3, 4, *bad, 1e4, None, ctypes.byref(out)) == _lib.E_INVALID
            checked += 1
            continue
        args = case_for(rid, tab.handle, other.handle, None)
        if args is None:
            continue
        if rid == "too_large":
            args = args[:-1] + (big.handle,)
        ok, got = call_can_use(*args)
        assert (ok, got) == (0, reason), (rid, got)
        checked += 1
    assert checked >= 9
    # the valid case passes (host-table mode skips the device-memory rule)
    q, k, qo, ko = fake_ptrs(2)
    assert call_can_use(qo, ko, q, k, _lib.DTYPE_BF16, SHAPE, tab.handle) == (1, "OK")
    assert call_can_use(None, None, q, k, _lib.DTYPE_BF16, SHAPE, tab.handle) == (1, "OK")
    assert call_can_use(qo, ko, q, k, _lib.DTYPE_F32, SHAPE, tab.handle) == (1, "OK")
    # fp32 pairs need 8-byte alignment, bf16 pairs 4-byte
    assert call_can_use(qo, ko, q + 4, k, _lib.DTYPE_F32, SHAPE, tab.handle) == (0, "ALIGN")
    assert call_can_use(qo, ko, q + 4, k, _lib.DTYPE_BF16, SHAPE, tab.handle) == (1, "OK")
    # q and k may alias each other (both are only read)
    assert call_can_use(qo, ko, q, q, _lib.DTYPE_BF16, SHAPE, tab.handle) == (1, "OK")
    # an output overlapping the other output
    assert call_can_use(qo, qo + 4, q, k, _lib.DTYPE_BF16, SHAPE, tab.handle) == (0, "OVERLAP")
    # just-touching ranges do not overlap
    nbytes = NUMEL * 2
    assert call_can_use(q + nbytes, q + 2 * nbytes, q, q, _lib.DTYPE_BF16, SHAPE, tab.handle) == (1, "OK")
    for t in (tab, other, big):
        t.close()


def test_split_odd_is_unreachable_through_tables_but_named():
    # tables cannot be built with an odd split, so SPLIT_ODD can only come from a corrupt handle;
    # the rule is still documented and has a reason string
    assert _lib.reason_string(_lib.REASON_CODES["SPLIT_ODD"]).startswith("each rope_dim_split")


def test_apply_refuses_in_host_table_mode():
    tab = rla.tables_build(2, 3, 4, SPLIT)
    q, k, qo, ko = fake_ptrs(2)
    st = L.ltx3drope_apply_qk(qo, ko, q, k, _lib.DTYPE_BF16, *SHAPE, tab.handle, None)
    assert st == _lib.E_UNSUPPORTED
    assert rla.stats()["rejected"] == 1
    assert rla.stats()["fast_launches"] == 0 and rla.stats()["plain_launches"] == 0
    tab.close()


def test_kernel_choice_rules():
    q, k, qo, ko = fake_ptrs(2)
    with rla.tables_build(2, 3, 4, (32, 48, 48)) as tab:
        shp = (1, 2, 3, 4, 16, 128)
        assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_BF16, *shp, tab.handle) == 1
        # 4-byte aligned but not 16-byte aligned -> plain
        assert L.ltx3drope_kernel_choice(qo, ko, q + 4, k, _lib.DTYPE_BF16, *shp, tab.handle) == 2
        # many heads (640 16-byte vectors per token) stay on the fast kernel
        shp_big = (1, 2, 3, 4, 40, 128)
        assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_BF16, *shp_big, tab.handle) == 1
        # head rows that are not a whole number of 16-byte vectors -> plain
        with rla.tables_build(2, 3, 4, (8, 8, 4)) as tab2:
            assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_BF16, 1, 2, 3, 4, 3, 20, tab2.handle) == 2
    with rla.tables_build(2, 3, 4, (2, 6, 4)) as tab:  # bf16 head row of 24 bytes: not whole vectors
        assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_BF16, 1, 2, 3, 4, 2, 12, tab.handle) == 2
        assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_F32, 1, 2, 3, 4, 2, 12, tab.handle) == 1
    with rla.tables_build(2, 3, 4, (4, 8, 4)) as tab:  # chunk widths not multiples of a vector's pairs
        assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_F32, 1, 2, 3, 4, 2, 16, tab.handle) == 1
        assert L.ltx3drope_kernel_choice(qo, ko, q, k, _lib.DTYPE_BF16, 1, 2, 3, 4, 2, 16, tab.handle) == 1
    # NULL outputs stand for fresh (aligned) outputs: only the inputs decide; one NULL is refused
    with rla.tables_build(2, 3, 4, (32, 48, 48)) as tab:
        shp = (1, 2, 3, 4, 16, 128)
        assert L.ltx3drope_kernel_choice(None, None, q, k, _lib.DTYPE_BF16, *shp, tab.handle) == 1
        assert L.ltx3drope_kernel_choice(None, None, q + 4, k, _lib.DTYPE_BF16, *shp, tab.handle) == 2
        assert L.ltx3drope_kernel_choice(qo, None, q, k, _lib.DTYPE_BF16, *shp, tab.handle) == _lib.E_UNSUPPORTED


# ---------------------------------------------------------------------------
# options and gate bookkeeping
# ---------------------------------------------------------------------------

def test_options_roundtrip_and_validation():
    for opt, vals in ((rla.OPT_PATH, (0, 1, 2)), (rla.OPT_GATE, (0, 1, 2)), (rla.OPT_LOG, (0, 1)),
                      (rla.OPT_FORCE_GATE_MISMATCH, (1, 0))):
        old = rla.get_option(opt)
        for v in vals:
            rla.set_option(opt, v)
            assert rla.get_option(opt) == v
        rla.set_option(opt, old)
    assert L.ltx3drope_set_option(rla.OPT_PATH, 3) == _lib.E_INVALID
    assert L.ltx3drope_set_option(99, 1) == _lib.E_INVALID
    assert L.ltx3drope_get_option(99) == _lib.E_INVALID


def test_gate_state_unseen_and_reset():
    rla.gate_reset()
    assert rla.gate_state(0, _lib.DTYPE_BF16, (1, 2, 3, 4, 2, 12), SPLIT) == "UNSEEN"


def test_copy_rejects_bad_arguments():
    assert L.ltx3drope_copy(None, None, 16, None) == _lib.E_INVALID
    assert L.ltx3drope_copy(1 << 32, (1 << 32) + 64, 15, None) == _lib.E_INVALID
    assert L.ltx3drope_copy(1 << 32, (1 << 32) + 8, 16, None) == _lib.E_INVALID


# ---------------------------------------------------------------------------
# shard placement and in-place aliasing (precheck only)
# ---------------------------------------------------------------------------

def call_can_use_shard(q_out, k_out, q, k, dtype, shape, shard, tab):
    reason = ctypes.c_int(-1)
    sh = None if shard is None else ctypes.byref(shard)
    ok = L.ltx3drope_can_use_shard(q_out, k_out, q, k, dtype, *shape, sh, tab, ctypes.byref(reason))
    return ok, _lib.REASONS[reason.value]


def test_shard_containment_rules():
    q, k, qo, ko = fake_ptrs(2)
    bf = _lib.DTYPE_BF16
    with rla.tables_build(8, 6, 5, SPLIT) as tab:
        local = (1, 2, 6, 5, 2, 12)
        assert call_can_use_shard(qo, ko, q, k, bf, local, _lib.Shard(6, 0, 0, 0, 0), tab.handle) == (1, "OK")
        assert call_can_use_shard(qo, ko, q, k, bf, local, _lib.Shard(7, 0, 0, 0, 0), tab.handle) == (0, "TABLE_GRID")
        assert call_can_use_shard(qo, ko, q, k, bf, local, _lib.Shard(-1, 0, 0, 0, 0), tab.handle) == (0, "TABLE_GRID")
        assert call_can_use_shard(qo, ko, q, k, bf, local, _lib.Shard(0, 1, 0, 0, 0), tab.handle) == (0, "TABLE_GRID")
        assert call_can_use_shard(qo, ko, q, k, bf, local, _lib.Shard(0, 0, 0, 0, 1), tab.handle) == (0, "TABLE_GRID")
        assert call_can_use_shard(qo, ko, q, k, bf, local, _lib.Shard(0, 0, 0, 2, 0), tab.handle) == (0, "TABLE_GRID")
        # spatial tiles: rows 2..4 and columns 1..3 of the 6x5 grid
        tile = (1, 8, 3, 3, 2, 12)
        assert call_can_use_shard(qo, ko, q, k, bf, tile, _lib.Shard(0, 2, 1, 0, 0), tab.handle) == (1, "OK")
        assert call_can_use_shard(qo, ko, q, k, bf, tile, _lib.Shard(0, 4, 1, 0, 0), tab.handle) == (0, "TABLE_GRID")
        assert call_can_use_shard(qo, ko, q, k, bf, tile, _lib.Shard(0, 2, 3, 0, 0), tab.handle) == (0, "TABLE_GRID")
        # a NULL descriptor means offsets 0: a sub-grid at the origin is accepted by the shard entry ...
        assert call_can_use_shard(qo, ko, q, k, bf, local, None, tab.handle) == (1, "OK")
        # ... but the unsharded entry keeps the page's exact grid rule
        assert call_can_use(qo, ko, q, k, bf, local, tab.handle) == (0, "TABLE_GRID")
        full = (1, 8, 6, 5, 2, 12)
        assert call_can_use(qo, ko, q, k, bf, full, tab.handle) == (1, "OK")


def test_inplace_aliasing_rules():
    q, k, qo, ko = fake_ptrs(2)
    bf = _lib.DTYPE_BF16
    with rla.tables_build(2, 3, 4, SPLIT) as tab:
        inpl = _lib.Shard(0, 0, 0, 1, 0)
        outp = _lib.Shard(0, 0, 0, 0, 0)
        assert call_can_use_shard(q, k, q, k, bf, SHAPE, inpl, tab.handle) == (1, "OK")
        assert call_can_use_shard(q, k, q, k, bf, SHAPE, outp, tab.handle) == (0, "OVERLAP")
        assert call_can_use_shard(q + 4, k, q, k, bf, SHAPE, inpl, tab.handle) == (0, "OVERLAP")  # partial
        assert call_can_use_shard(q, ko, q, k, bf, SHAPE, inpl, tab.handle) == (1, "OK")  # only Q in place
        assert call_can_use_shard(k, q, q, k, bf, SHAPE, inpl, tab.handle) == (0, "OVERLAP")  # crossed
        assert call_can_use_shard(q, q, q, q, bf, SHAPE, inpl, tab.handle) == (0, "OVERLAP")  # q aliases k
        st = L.ltx3drope_apply_qk_shard(q, k, q, k, bf, *SHAPE, ctypes.byref(_lib.Shard(0, 0, 0, 3, 0)), tab.handle,
                                         None)
        assert st == _lib.E_TABLE_MISMATCH


# ---------------------------------------------------------------------------
# rotate-half RoPE precheck (rules decided before any device-memory query)
# ---------------------------------------------------------------------------

def call_neox_can_use(q_out, k_out, q, k, dtype, tokens, qh, kh, D, pos, cache, cdt, maxp):
    reason = ctypes.c_int(-1)
    ok = L.ltx3drope_neox_can_use(q_out, k_out, q, k, dtype, tokens, qh, kh, D, pos, cache, cdt, maxp,
                                  ctypes.byref(reason))
    return ok, _lib.REASONS[reason.value]


def test_neox_precheck_rules():
    base = 1 << 32
    gap = 1 << 24
    q, k, qo, ko, pos, cache = (base + i * gap for i in range(6))
    bf, f32 = _lib.DTYPE_BF16, _lib.DTYPE_F32
    good = (qo, ko, q, k, bf, 16, 4, 2, 64, pos, cache, f32, 128)
    assert call_neox_can_use(*good[:9], None, *good[10:]) == (0, "NULLPTR")
    assert call_neox_can_use(*good[:4], 5, *good[5:]) == (0, "DTYPE")
    assert call_neox_can_use(*good[:11], 9, good[12]) == (0, "DTYPE")
    assert call_neox_can_use(*good[:5], -1, *good[6:]) == (0, "NONPOSITIVE_DIM")
    # no tokens: an empty call, valid whenever the other sizes and the dtypes are (pointers unread)
    assert call_neox_can_use(*good[:5], 0, *good[6:]) == (1, "OK")
    assert call_neox_can_use(None, None, None, None, bf, 0, 4, 2, 64, None, None, f32, 128) == (1, "OK")
    assert call_neox_can_use(None, None, None, None, bf, 0, 4, 2, 63, None, None, f32, 128) == (0, "SPLIT_ODD")
    assert call_neox_can_use(None, None, None, None, bf, 0, 0, 2, 64, None, None, f32, 128) == (0, "NONPOSITIVE_DIM")
    assert call_neox_can_use(None, None, None, None, bf, 0, 4, 2, 64, None, None, 7, 128) == (0, "DTYPE")
    assert call_neox_can_use(None, None, None, None, bf, 0, 4, 2, 64, None, None, f32, 1 << 31) == (0, "TOO_LARGE")
    assert call_neox_can_use(*good[:12], 0) == (0, "NONPOSITIVE_DIM")
    assert call_neox_can_use(*good[:8], 63, *good[9:]) == (0, "SPLIT_ODD")
    assert call_neox_can_use(qo + 1, *good[1:]) == (0, "ALIGN")
    assert call_neox_can_use(*good[:9], pos + 4, *good[10:]) == (0, "ALIGN")
    assert call_neox_can_use(*good[:10], cache + 2, *good[11:]) == (0, "ALIGN")
    assert call_neox_can_use(*good[:5], 1 << 20, 1 << 10, 2, 64, *good[9:]) == (0, "TOO_LARGE")
    # the size limit: fewer than 2^32 elements per tensor (2^25 tokens x 128 = 2^32 is refused)
    far = [base + i * (1 << 40) for i in range(6)]
    big = (far[0], far[1], far[2], far[3], bf, 1 << 25, 1, 1, 128, far[4], far[5], f32, 128)
    assert call_neox_can_use(*big) == (0, "TOO_LARGE")
    assert call_neox_can_use(*big[:8], 126, *big[9:])[1] in ("NOT_DEVICE_PTR", "OK")  # past the host rules
    assert call_neox_can_use(q + 64, *good[1:]) == (0, "OVERLAP")        # partial overlap of q_out and q
    assert call_neox_can_use(qo, cache + 16, *good[2:]) == (0, "OVERLAP")  # k_out over the cache
    assert call_neox_can_use(pos, *good[1:]) == (0, "OVERLAP")             # q_out over the positions
    assert call_neox_can_use(k, *good[1:]) == (0, "OVERLAP")               # q_out over k
    # exact in-place aliasing passes every host rule (device memory is checked last)
    ok, reason = call_neox_can_use(q, k, *good[2:])
    assert reason in ("NOT_DEVICE_PTR", "OK")
    # both outputs NULL: fresh outputs, only the inputs are checked; one NULL output is refused
    assert call_neox_can_use(None, None, *good[2:])[1] in ("NOT_DEVICE_PTR", "OK")
    assert call_neox_can_use(None, None, q + 1, *good[3:]) == (0, "ALIGN")
    assert call_neox_can_use(None, None, *good[2:5], 1 << 20, 1 << 10, 2, 64, *good[9:]) == (0, "TOO_LARGE")
    assert call_neox_can_use(qo, None, *good[2:]) == (0, "NULLPTR")


# ---------------------------------------------------------------------------
# LTX DiT RoPE frequency grid (host computation, host output)
# ---------------------------------------------------------------------------

def test_dit_freq_grid_rejects_bad_arguments():
    n = ctypes.c_int64(-1)
    for args in ((0.0, 64, 2), (-1.0, 64, 2), (float("inf"), 64, 2), (float("nan"), 64, 2), (1e-39, 64, 2),
                 (3.5e38, 64, 2), (1e4, -1, 2), (1e4, 64, 0), (1e4, (1 << 24) + 1, 1)):
        assert L.ltx3drope_dit_freq_grid(*args, 1, None, None, ctypes.byref(n)) == _lib.E_INVALID
    assert L.ltx3drope_dit_freq_grid(1e4, 64, 2, 1, None, None, ctypes.byref(n)) == _lib.E_INVALID  # NULL out
    assert L.ltx3drope_dit_freq_grid(1e4, 1, 2, 1, None, None, ctypes.byref(n)) == _lib.OK and n.value == 0
    host = (ctypes.c_float * 32)()
    assert L.ltx3drope_dit_freq_grid(1e4, 64, 2, 1, host, None, ctypes.byref(n)) in (_lib.E_UNSUPPORTED, _lib.E_HIP)


def test_binding_refuses_host_tensors_and_bad_patch_sizes_before_any_call():
    """The binding's own argument checks (no library call is made for these)."""
    import torch

    q = torch.zeros(1, 2, 2, 2, 1, 6)
    with pytest.raises(rla.Ltx3dRopeUnsupported) as e:
        rla.forward_pair(q, q.clone(), (2, 2, 2))
    assert e.value.reason == "NOT_DEVICE_PTR"
    assert rla.can_use(q, q.clone(), None) == (False, "NOT_DEVICE_PTR")
    with pytest.raises(rla.Ltx3dRopeUnsupported):
        rla.patchify(torch.zeros(1, 1, 1, 4, 4), 2)  # host tensor
    for p in (0, -2):
        with pytest.raises(ValueError):
            rla.unpatchify(torch.zeros(1, 4, 1, 2, 2), p)
    assert rla.stats()["rejected"] == 0  # nothing reached the library


def test_size_limit_is_2_to_the_32_elements_per_batch_element():
    """A batch element of the 3D RoPE holds up to 2^32 - 1 elements: just below passes the host
    rules, 2^32 is TOO_LARGE, and so is any single size of 2^31 or more.  A tensor of 2^32
    elements or more made of smaller batch elements passes (it runs as several launches)."""
    split = (16, 16, 32)
    with rla.tables_build(1, 1, 1 << 20, split) as tab:
        base = 1 << 20
        args = (base + (1 << 40), base + (2 << 40), base, base + (4 << 40), _lib.DTYPE_BF16)
        assert call_can_use(*args, (1, 1, 1, 1 << 20, 63, 64), tab.handle) == (1, "OK")
        assert call_can_use(*args, (1, 1, 1, 1 << 20, 64, 64), tab.handle) == (0, "TOO_LARGE")
        assert call_can_use(*args, (3, 1, 1, 1 << 20, 40, 64), tab.handle) == (1, "OK")  # 3 x 2.7 G elements
    with rla.tables_build(1, 1, 1, (2, 2, 2)) as tab:
        assert call_can_use(*args, (1 << 31, 1, 1, 1, 1, 6), tab.handle) == (0, "TOO_LARGE")
        assert call_can_use(*args, ((1 << 31) - 1, 1, 1, 1, 1, 6), tab.handle) == (1, "OK")
        assert call_can_use(*args, (1 << 30, 1, 1, 1, 1 << 20, 6), tab.handle) == (0, "TOO_LARGE")  # 2^52 in all


def test_empty_calls_launch_nothing():
    """Zero tokens (rotate-half RoPE) or a zero size (patchify) is a successful call that reads no
    pointer and launches nothing; negative sizes stay invalid."""
    bf, f32 = _lib.DTYPE_BF16, _lib.DTYPE_F32
    before = rla.stats()
    assert L.ltx3drope_neox_apply_qk(None, None, None, None, bf, 0, 4, 2, 64, None, None, f32, 128, None) == _lib.OK
    assert L.ltx3drope_neox_apply_qk(None, None, None, None, bf, -1, 4, 2, 64, None, None, f32, 128,
                                     None) == _lib.E_UNSUPPORTED
    for fn in (L.ltx3drope_patchify, L.ltx3drope_unpatchify):
        for sizes in ((0, 3, 5, 8, 8), (1, 0, 5, 8, 8), (1, 3, 0, 8, 8), (1, 3, 5, 0, 8), (1, 3, 5, 8, 0)):
            assert fn(None, None, 2, *sizes, 2, None) == _lib.OK
        assert fn(None, None, 2, 1, 3, 5, 8, -8, 2, None) == _lib.E_INVALID
        assert fn(None, None, 2, 0, 3, 5, 8, 6, 4, None) == _lib.E_INVALID  # W not a multiple of p
        assert fn(None, None, 3, 0, 3, 5, 8, 8, 2, None) == _lib.E_INVALID  # element size
        assert fn(None, None, 2, 1, 3, 5, 8, 8, 2, None) == _lib.E_INVALID  # NULL pointers of a real call
    after = rla.stats()
    assert after["fast_launches"] == before["fast_launches"] and after["plain_launches"] == before["plain_launches"]
