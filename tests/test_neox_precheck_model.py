"""Property test of the rotate-half RoPE precheck (ltx3drope_neox_can_use) against a model of its
documented rule order, on the CPU.

The model restates the rules of include/ltx3drope.h for the rotate-half RoPE in their documented
order (the first that fails names the reason), for empty calls and for calls with tokens.
Hypothesis draws sizes, dtypes and pointer layouts around each rule's boundary.  The device-memory
rules come last; on a host without device memory at these fake addresses they report
NOT_DEVICE_PTR, which is what the model expects of a call that passes every host rule.
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
BASE = 1 << 56  # fake addresses, never dereferenced by the host rules
STRIDE = 1 << 50
F32, BF16 = _lib.DTYPE_F32, _lib.DTYPE_BF16
LIM, SIZE_LIM = 1 << 32, 1 << 31


def model(q_out, k_out, q, k, dtype, tokens, qh, kh, D, pos, cache, cdt, maxp):
    """The documented verdict (a reason name)."""
    dtypes_ok = dtype in (F32, BF16) and cdt in (F32, BF16)
    if tokens == 0:
        if not dtypes_ok:
            return "DTYPE"
        if min(qh, kh, D, maxp) <= 0:
            return "NONPOSITIVE_DIM"
        if D % 2:
            return "SPLIT_ODD"
        if max(qh, kh, D, maxp) >= SIZE_LIM or maxp * D >= LIM:
            return "TOO_LARGE"
        return "OK"
    outputs = q_out is not None or k_out is not None
    if (outputs and (q_out is None or k_out is None)) or None in (q, k, pos, cache):
        return "NULLPTR"
    if not dtypes_ok:
        return "DTYPE"
    if min(tokens, qh, kh, D, maxp) <= 0:
        return "NONPOSITIVE_DIM"
    if D % 2:
        return "SPLIT_ODD"
    es = 4 if dtype == F32 else 2
    cs = 4 if cdt == F32 else 2
    if any(p is not None and p % es for p in (q_out, k_out, q, k)) or cache % cs or pos % 8:
        return "ALIGN"

    def fits(*fs):
        n = 1
        for f in fs:
            if f >= SIZE_LIM:
                return False
            n *= f
        return n < LIM

    if not (fits(tokens, qh, D) and fits(tokens, kh, D) and fits(maxp, D)):
        return "TOO_LARGE"
    if outputs:
        qb, kb, pb, cb = tokens * qh * D * es, tokens * kh * D * es, tokens * 8, maxp * D * cs

        def overlap(a, an, b, bn):
            return a < b + bn and b < a + an

        if ((q_out != q and overlap(q_out, qb, q, qb)) or overlap(q_out, qb, k, kb) or overlap(k_out, kb, q, qb)
                or (k_out != k and overlap(k_out, kb, k, kb)) or overlap(q_out, qb, k_out, kb)):
            return "OVERLAP"
        for o, ob in ((q_out, qb), (k_out, kb)):
            if overlap(o, ob, pos, pb) or overlap(o, ob, cache, cb):
                return "OVERLAP"
    return "NOT_DEVICE_PTR"


def usually(good, rare):
    """Mostly a valid value (so that draws reach the later rules), sometimes one at or past a
    rule's boundary."""
    return st.integers(0, 9).flatmap(lambda r: good if r < 8 else rare)


BIG = [1 << 20, (1 << 31) - 1, 1 << 31, 1 << 32]


@st.composite
def cases(draw):
    dtype = draw(usually(st.sampled_from([F32, BF16]), st.sampled_from([2, -1])))
    cdt = draw(usually(st.sampled_from([F32, BF16]), st.sampled_from([5])))
    if draw(st.integers(0, 4)) == 0:
        # at the size limits: 2^32 elements in a tensor or in the cache (refused), one less (accepted)
        tokens = draw(st.sampled_from([1 << 25, (1 << 25) - 1, 1 << 24, 0]))
        qh, kh, D = draw(st.sampled_from([1, 2])), draw(st.sampled_from([1, 2])), 128
        maxp = draw(st.sampled_from([1 << 25, (1 << 25) - 1, 4096]))
    else:
        tokens = draw(usually(st.integers(1, 64), st.sampled_from([0, 0, -1, 1 << 20, 1 << 25, 1 << 31])))
        qh = draw(usually(st.integers(1, 16), st.sampled_from([0, -2] + BIG)))
        kh = draw(usually(st.integers(1, 8), st.sampled_from([0, -1] + BIG)))
        D = draw(usually(st.sampled_from([2, 16, 64, 128, 256]), st.sampled_from([0, -2, 63, 1 << 20, 1 << 31])))
        maxp = draw(usually(st.integers(1, 4096), st.sampled_from([0, -1, 1 << 24, (1 << 31) - 1, 1 << 31])))
    q = BASE + draw(usually(st.just(0), st.sampled_from([1, 2, 4])))
    k = BASE + STRIDE + draw(usually(st.just(0), st.sampled_from([2, 6])))
    pos = BASE + 2 * STRIDE + draw(usually(st.just(0), st.sampled_from([4, 2])))
    cache = BASE + 3 * STRIDE + draw(usually(st.just(0), st.sampled_from([2, 6])))
    fresh_q, fresh_k = BASE + 4 * STRIDE, BASE + 5 * STRIDE
    kind = draw(st.sampled_from(["fresh", "fresh", "fresh", "none", "in_place", "q_out_over_q", "q_out_over_k",
                                 "k_out_over_q", "k_out_near_k", "outputs_overlap", "over_positions",
                                 "over_cache", "one_null", "null_input"]))
    q_out = k_out = None
    if kind == "fresh":
        q_out, k_out = fresh_q, fresh_k
    elif kind == "in_place":
        q_out, k_out = q, draw(st.sampled_from([k, fresh_k]))
    elif kind == "q_out_over_q":
        q_out, k_out = q + draw(st.sampled_from([-64, 64, 1 << 16])), fresh_k
    elif kind == "q_out_over_k":
        q_out, k_out = k + draw(st.sampled_from([0, 64])), fresh_k
    elif kind == "k_out_over_q":
        q_out, k_out = fresh_q, q + draw(st.sampled_from([0, 64]))
    elif kind == "k_out_near_k":
        q_out, k_out = fresh_q, k + draw(st.sampled_from([-64, 64]))
    elif kind == "outputs_overlap":
        q_out, k_out = fresh_q, fresh_q + draw(st.sampled_from([0, 64, 1 << 12]))
    elif kind == "over_positions":
        q_out, k_out = draw(st.sampled_from([(pos - 64, fresh_k), (fresh_q, pos + 64)]))
    elif kind == "over_cache":
        q_out, k_out = draw(st.sampled_from([(cache + 64, fresh_k), (fresh_q, cache - 64)]))
    elif kind == "one_null":
        q_out = fresh_q
    elif kind == "null_input":
        which = draw(st.integers(0, 3))
        q, k, pos, cache = [None if i == which else v for i, v in enumerate((q, k, pos, cache))]
        q_out, k_out = fresh_q, fresh_k
    return q_out, k_out, q, k, dtype, tokens, qh, kh, D, pos, cache, cdt, maxp


def library(q_out, k_out, q, k, dtype, tokens, qh, kh, D, pos, cache, cdt, maxp):
    reason = ctypes.c_int(-1)
    ok = L.ltx3drope_neox_can_use(q_out, k_out, q, k, dtype, tokens, qh, kh, D, pos, cache, cdt, maxp,
                                  ctypes.byref(reason))
    return ok, _lib.REASONS[reason.value]


SETTINGS = dict(max_examples=1500, deadline=None, derandomize=True, database=None,
                suppress_health_check=list(HealthCheck))


@settings(**SETTINGS)
@given(cases())
def test_neox_precheck_matches_its_documented_rules(case):
    ok, got = library(*case)
    want = model(*case)
    if want == "NOT_DEVICE_PTR":
        # past every host rule: device memory is checked last (a GPU host may hold memory there)
        assert got in ("NOT_DEVICE_PTR", "TABLE_DEVICE", "EXTENT", "OK"), (case, got)
    else:
        assert got == want, (case, got, want)
        assert ok == (1 if want == "OK" else 0)


def test_model_reaches_every_reason():
    """The strategy reaches every rule (guards against a model that agrees only vacuously)."""
    seen = set()

    @settings(**SETTINGS)
    @given(cases())
    def collect(case):
        seen.add(model(*case))

    collect()
    assert seen >= {"OK", "NULLPTR", "DTYPE", "NONPOSITIVE_DIM", "SPLIT_ODD", "ALIGN", "TOO_LARGE", "OVERLAP",
                    "NOT_DEVICE_PTR"}, seen
