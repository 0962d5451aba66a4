"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's code path: each checks the oracle
against a closed form, an arbitrary-precision evaluation, a library routine
(torch's CPU bf16 cast, numpy complex arithmetic) or a brute-force
recomputation that addresses elements through explicit strides.  The last
group plants plausible mistakes into the oracle (on the CPU) and checks that
at least one pin catches each of them.
"""
from __future__ import annotations

import math
import struct

import numpy as np
import pytest
import torch

import oracle
import oracle.rope as orc
import workloads
from tests import exact_trig

BASE = 10000.0


# ---------------------------------------------------------------------------
# pin functions (each raises AssertionError on a mismatch)
# ---------------------------------------------------------------------------

def pin_inv_freq_closed_forms():
    # base**(-2i/d) is an exact power of ten whenever (2i/d)*log10(base) is an integer
    cases = [  # (base, dim, i, value)
        (10000.0, 16, 0, 1.0), (10000.0, 16, 2, 0.1), (10000.0, 16, 4, 0.01), (10000.0, 16, 6, 0.001),
        (10000.0, 32, 4, 0.1), (10000.0, 32, 8, 0.01), (10000.0, 32, 12, 0.001),
        (10000.0, 48, 6, 0.1), (10000.0, 48, 12, 0.01), (10000.0, 48, 18, 0.001),
        (10000.0, 96, 12, 0.1), (10000.0, 96, 24, 0.01), (100.0, 8, 2, 0.1), (100.0, 4, 1, 0.1),
    ]
    for base, dim, i, value in cases:
        got = orc.inv_freqs(dim, base)[i]
        assert math.isclose(got, value, rel_tol=2 ** -51), (base, dim, i, got, value)
    for dim in (8, 16, 32, 48, 96, 128):
        om = orc.inv_freqs(dim, BASE)
        assert len(om) == dim // 2
        assert om[0] == 1.0
        assert all(a > b for a, b in zip(om, om[1:]))
        ratio = BASE ** (-2.0 / dim)
        for a, b in zip(om, om[1:]):
            assert math.isclose(b / a, ratio, rel_tol=1e-13)


def pin_tables_exact(length, dim, base=BASE, entries=None):
    """Oracle tables equal the correctly rounded fp32 cos/sin of p*base**(-2i/d)."""
    cos, sin = orc.axis_tables(length, dim, base)
    assert cos.shape == (length, dim // 2) and sin.shape == (length, dim // 2)
    assert cos.dtype == np.float32 and sin.dtype == np.float32
    if entries is None:
        ec, es, amb = exact_trig.exact_axis_tables(length, dim, base)
        ok = (cos == ec) & (sin == es)
        assert np.all(ok | amb), np.argwhere(~(ok | amb))[:5]
    else:
        for p, i in entries:
            c, s, amb = exact_trig.table_entry(base, dim, p, i)
            assert amb or (cos[p, i] == c and sin[p, i] == s), (p, i, cos[p, i], c, sin[p, i], s)


def pin_table_closed_forms(length, dim, base=BASE):
    cos, sin = orc.axis_tables(length, dim, base)
    # position 0: angle 0 for every column
    assert np.all(cos[0] == np.float32(1.0)) and np.all(sin[0] == np.float32(0.0))
    # column 0: omega_0 = 1, so the angle is the position itself
    for p in range(length):
        assert cos[p, 0] == np.float32(math.cos(p)) and sin[p, 0] == np.float32(math.sin(p))
    c = cos.astype(np.float64)
    s = sin.astype(np.float64)
    r = c * c + s * s
    assert np.all(np.abs(r - 1.0) <= 2.0 ** -22), np.max(np.abs(r - 1.0))


def _brute_force_qk(q, k, dtype, split, base, offsets=(0, 0, 0)):
    """Element-by-element rotation through explicit strides, with the tables taken
    from the arbitrary-precision evaluation and bf16 rounding from torch.  With
    offsets the tensor is a shard whose first frame/row/column sits at those
    global coordinates."""
    B, T, H, W, heads, D = q.shape
    dt, dh, dw = split
    t0, h0, w0 = offsets
    tabs = [exact_trig.exact_axis_tables(L, d, base) for L, d in ((T + t0, dt), (H + h0, dh), (W + w0, dw))]
    for _, _, amb in tabs:
        assert not amb.any()
    outs = []
    for x in (q, k):
        flat = x.reshape(-1)
        res = np.empty(flat.size, dtype=np.float32)
        for b in range(B):
            for t in range(T):
                for h in range(H):
                    for w in range(W):
                        for hd in range(heads):
                            row = ((((b * T + t) * H + h) * W + w) * heads + hd) * D
                            for j in range(D // 2):
                                if j < dt // 2:
                                    axis, col, pos = 0, j, t + t0
                                elif j < (dt + dh) // 2:
                                    axis, col, pos = 1, j - dt // 2, h + h0
                                else:
                                    axis, col, pos = 2, j - (dt + dh) // 2, w + w0
                                c = tabs[axis][0][pos, col]
                                s = tabs[axis][1][pos, col]
                                if dtype == oracle.BF16:
                                    e = struct.unpack("<f", struct.pack("<I", int(flat[row + 2 * j]) << 16))[0]
                                    o = struct.unpack("<f", struct.pack("<I", int(flat[row + 2 * j + 1]) << 16))[0]
                                    e, o = np.float32(e), np.float32(o)
                                else:
                                    e, o = flat[row + 2 * j], flat[row + 2 * j + 1]
                                res[row + 2 * j] = np.float32(np.float32(e * c) - np.float32(o * s))
                                res[row + 2 * j + 1] = np.float32(np.float32(e * s) + np.float32(o * c))
        if dtype == oracle.BF16:
            out = torch.from_numpy(res).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            out = res
        outs.append(out.reshape(x.shape))
    return outs


def pin_brute_force(shape, dtype, split, seed, base=BASE, offsets=(0, 0, 0)):
    q, k = workloads.generate_custom(shape, dtype, seed)
    qo, ko = orc.rope3d_qk(q, k, dtype, split, base, offsets=offsets)
    bq, bk = _brute_force_qk(q, k, dtype, split, base, offsets)
    assert qo.dtype == q.dtype and ko.dtype == k.dtype
    np.testing.assert_array_equal(qo.view(np.uint32 if dtype == oracle.F32 else np.uint16),
                                  bq.view(np.uint32 if dtype == oracle.F32 else np.uint16))
    np.testing.assert_array_equal(ko.view(np.uint32 if dtype == oracle.F32 else np.uint16),
                                  bk.view(np.uint32 if dtype == oracle.F32 else np.uint16))


def pin_unit_vectors(grid, split, heads=2, base=BASE):
    """Pairs (1, 0) come out as (cos, sin) and pairs (0, 1) as (-sin, cos): the
    output is the table gathered through the token and pair mapping."""
    T, H, W = grid
    D = sum(split)
    shape = (1, T, H, W, heads, D)
    one0 = np.zeros(shape, np.float32)
    one0[..., 0::2] = 1.0
    zero1 = np.zeros(shape, np.float32)
    zero1[..., 1::2] = 1.0
    tabs = orc.grid_tables(T, H, W, split, base)
    a, _ = orc.rope3d_qk(one0, one0, oracle.F32, split, base)
    b, _ = orc.rope3d_qk(zero1, zero1, oracle.F32, split, base)
    dt, dh, dw = split
    for t in range(T):
        for h in range(H):
            for w in range(W):
                for hd in range(heads):
                    c = np.concatenate([tabs[0][0][t], tabs[1][0][h], tabs[2][0][w]])
                    s = np.concatenate([tabs[0][1][t], tabs[1][1][h], tabs[2][1][w]])
                    np.testing.assert_array_equal(a[0, t, h, w, hd, 0::2], c)
                    np.testing.assert_array_equal(a[0, t, h, w, hd, 1::2], s)
                    np.testing.assert_array_equal(b[0, t, h, w, hd, 0::2], -s)
                    np.testing.assert_array_equal(b[0, t, h, w, hd, 1::2], c)
    # rotation by +theta: for the first non-zero position the sine is positive
    if H > 1:
        assert a[0, 0, 1, 0, 0, dt + 1] > 0  # h = 1, first h column: sin(1) > 0


def pin_identity_at_origin(dtype, seed=11):
    """A 1x1x1 grid has only position 0: the output equals the input by value."""
    shape = (2, 1, 1, 1, 3, 24)
    q, k = workloads.generate_custom(shape, dtype, seed)
    qo, ko = orc.rope3d_qk(q, k, dtype, (8, 8, 8), BASE)
    np.testing.assert_array_equal(orc.to_f32(qo, dtype), orc.to_f32(q, dtype))
    np.testing.assert_array_equal(orc.to_f32(ko, dtype), orc.to_f32(k, dtype))


def pin_zero_sections_unchanged(dtype, seed=12):
    """Tokens at h = w = 0 leave the h and w channels unchanged (by value)."""
    shape = (1, 3, 2, 2, 2, 24)
    split = (8, 8, 8)
    q, k = workloads.generate_custom(shape, dtype, seed)
    qo, _ = orc.rope3d_qk(q, k, dtype, split, BASE)
    np.testing.assert_array_equal(orc.to_f32(qo[:, :, 0, 0, :, 8:], dtype), orc.to_f32(q[:, :, 0, 0, :, 8:], dtype))
    # and t = 0 leaves the t channels unchanged everywhere
    np.testing.assert_array_equal(orc.to_f32(qo[:, 0, :, :, :, :8], dtype), orc.to_f32(q[:, 0, :, :, :, :8], dtype))


def pin_norm_and_round_trip(seed=13):
    shape = (1, 5, 6, 7, 3, 48)
    split = (16, 16, 16)
    q, k = workloads.generate_custom(shape, oracle.F32, seed)
    qo, ko = orc.rope3d_qk(q, k, oracle.F32, split, BASE)
    for x, y in ((q, qo), (k, ko)):
        n_in = np.hypot(x[..., 0::2].astype(np.float64), x[..., 1::2].astype(np.float64))
        n_out = np.hypot(y[..., 0::2].astype(np.float64), y[..., 1::2].astype(np.float64))
        assert np.all(np.abs(n_out - n_in) <= 1e-6 * n_in), np.max(np.abs(n_out - n_in) / n_in)
    tabs = orc.grid_tables(5, 6, 7, split, BASE)
    inv = tuple((c, -s) for c, s in tabs)
    back = orc.rope3d(qo, oracle.F32, split, BASE, tables=inv)
    n_in = np.repeat(np.hypot(q[..., 0::2].astype(np.float64), q[..., 1::2].astype(np.float64)), 2, axis=-1)
    assert np.all(np.abs(back.astype(np.float64) - q) <= 1e-6 * n_in)


def pin_complex_product_bound(seed=14):
    """Each output pair is within the fp32 rounding bound of the exact complex
    product (e + i o)(c + i s), evaluated in complex128 with the table values."""
    shape = (2, 3, 4, 5, 2, 40)
    split = (12, 16, 12)
    q, k = workloads.generate_custom(shape, oracle.F32, seed)
    qo, _ = orc.rope3d_qk(q, k, oracle.F32, split, BASE)
    tabs = orc.grid_tables(3, 4, 5, split, BASE)
    t_i, h_i, w_i = np.meshgrid(np.arange(3), np.arange(4), np.arange(5), indexing="ij")
    cos = np.concatenate([tabs[0][0][t_i], tabs[1][0][h_i], tabs[2][0][w_i]], axis=-1)[None, :, :, :, None, :]
    sin = np.concatenate([tabs[0][1][t_i], tabs[1][1][h_i], tabs[2][1][w_i]], axis=-1)[None, :, :, :, None, :]
    z = q[..., 0::2].astype(np.float64) + 1j * q[..., 1::2].astype(np.float64)
    rot = cos.astype(np.float64) + 1j * sin.astype(np.float64)
    exact = z * rot
    e, o = np.abs(z.real), np.abs(z.imag)
    c, s = np.abs(rot.real), np.abs(rot.imag)
    u = 2.0 ** -24
    bound_re = (e * c + o * s) * 2 * u + np.abs(exact.real) * u
    bound_im = (e * s + o * c) * 2 * u + np.abs(exact.imag) * u
    assert np.all(np.abs(qo[..., 0::2] - exact.real) <= bound_re)
    assert np.all(np.abs(qo[..., 1::2] - exact.imag) <= bound_im)


def pin_shard_is_slab_of_full(full_shape, split, offsets, local, seed):
    """Rotating a slab of a tensor as a shard (with its offsets into the full grid) gives
    exactly that slab of the full tensor's result."""
    q, k = workloads.generate_custom(full_shape, oracle.BF16, seed)
    fq, fk = orc.rope3d_qk(q, k, oracle.BF16, split)
    (t0, h0, w0), (tl, hl, wl) = offsets, local
    sl = (slice(None), slice(t0, t0 + tl), slice(h0, h0 + hl), slice(w0, w0 + wl))
    sq, sk = np.ascontiguousarray(q[sl]), np.ascontiguousarray(k[sl])
    oq, ok = orc.rope3d_qk(sq, sk, oracle.BF16, split, offsets=offsets, grid=full_shape[1:4])
    np.testing.assert_array_equal(oq, fq[sl])
    np.testing.assert_array_equal(ok, fk[sl])
    ids = np.array([0, 3, sq.shape[0] * tl * hl * wl - 1])
    np.testing.assert_array_equal(orc.rope3d_sampled(sq, oracle.BF16, split, ids, offsets=offsets, grid=full_shape[1:4]),
                                  oq.reshape(-1, *sq.shape[4:])[ids])


def pin_sampled_equals_full(seed=15):
    shape = (2, 3, 4, 5, 2, 24)
    split = (8, 8, 8)
    q, _ = workloads.generate_custom(shape, oracle.BF16, seed)
    full = orc.rope3d(q, oracle.BF16, split, BASE).reshape(-1, 2, 24)
    ids = np.array([0, 7, 33, 59, 60, 119])
    np.testing.assert_array_equal(orc.rope3d_sampled(q, oracle.BF16, split, ids, BASE), full[ids])


def _bf16_patterns():
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    rnd = np.random.Generator(np.random.PCG64(99)).integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd]).view(np.float32)


def pin_bf16_cast():
    x = _bf16_patterns()
    ours = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(orc.bf16_bits_to_f32(ours[nan])))
    # closed-form properties: exact on bf16 values, ties to even, widening is exact
    allb = np.arange(65536, dtype=np.uint16)
    w = orc.bf16_bits_to_f32(allb)
    fin = ~np.isnan(w)
    np.testing.assert_array_equal(orc.f32_to_bf16_bits(w)[fin], allb[fin])
    tie = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x00018000], np.uint32).view(np.float32)
    np.testing.assert_array_equal(orc.f32_to_bf16_bits(tie), np.array([0x3F80, 0x3F82, 0xBF80, 0x0000, 0x0002], np.uint16))
    assert orc.f32_to_bf16_bits(np.array([3.4e38], np.float32))[0] == 0x7F80
    assert orc.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0] == 0xFF80


def pin_nan_canonical():
    """A NaN result is the canonical quiet NaN in both dtypes (0x7FC00000, 0x7FC0), whatever the
    sign and payload of the NaN that caused it; an infinity times a zero table entry (sin 0 at
    position 0) is a NaN too.  Every other element is untouched by the rule."""
    shape, split = (1, 2, 2, 2, 1, 12), (4, 4, 4)
    rng = np.random.Generator(np.random.PCG64(41))
    n = int(np.prod(shape))
    idx = rng.choice(n, 24, replace=False)
    f32 = rng.standard_normal(n).astype(np.float32)
    f32.view(np.uint32)[idx] = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF812345, 0x7FFFFFFF, 0x7FA00000],
                                        np.uint32)[np.arange(24) % 6]
    bf = orc.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    bf[idx] = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFF92, 0x7FFF, 0xFFA3], np.uint16)[np.arange(24) % 6]
    for dtype, x, canon in ((oracle.F32, f32, 0x7FC00000), (oracle.BF16, bf, 0x7FC0)):
        x = x.reshape(shape).copy()
        x.reshape(-1)[1] = np.float32(np.inf) if dtype == oracle.F32 else np.uint16(0x7F80)  # odd element, origin
        out = orc.rope3d(x, dtype, split, BASE)
        raw = out.view(np.uint32) if dtype == oracle.F32 else out
        nan = np.isnan(orc.to_f32(out, dtype))
        assert nan.sum() >= 24 and nan.reshape(-1)[0], int(nan.sum())
        assert np.all(raw[nan] == canon), [hex(v) for v in raw[nan][:4]]


ALL_PINS = [
    ("inv_freq", pin_inv_freq_closed_forms),
    ("tables_exact", lambda: (pin_tables_exact(4, 16), pin_tables_exact(5, 24), pin_tables_exact(3, 12))),
    ("table_closed_forms", lambda: pin_table_closed_forms(6, 16)),
    ("unit_vectors", lambda: pin_unit_vectors((2, 3, 4), (4, 8, 6))),
    ("identity", lambda: (pin_identity_at_origin(oracle.F32), pin_identity_at_origin(oracle.BF16))),
    ("zero_sections", lambda: pin_zero_sections_unchanged(oracle.BF16)),
    ("norm_round_trip", pin_norm_and_round_trip),
    ("complex_bound", pin_complex_product_bound),
    ("brute_f32", lambda: pin_brute_force((1, 2, 3, 2, 2, 16), oracle.F32, (4, 8, 4), 21)),
    ("brute_bf16", lambda: pin_brute_force((2, 2, 2, 3, 1, 12), oracle.BF16, (4, 4, 4), 22)),
    ("bf16_cast", pin_bf16_cast),
    ("brute_shard", lambda: pin_brute_force((1, 2, 2, 3, 1, 12), oracle.BF16, (4, 4, 4), 25, offsets=(3, 1, 2))),
    ("shard_slab", lambda: pin_shard_is_slab_of_full((2, 6, 5, 7, 2, 24), (8, 8, 8), (2, 1, 3), (3, 3, 4), 26)),
    ("nan_canonical", pin_nan_canonical),
]


# ---------------------------------------------------------------------------
# the pins themselves
# ---------------------------------------------------------------------------

def test_inv_freq_closed_forms():
    pin_inv_freq_closed_forms()


@pytest.mark.parametrize("length,dim", [(2, 16), (4, 16), (32, 32), (17, 32), (5, 48), (9, 96)])
def test_tables_match_exact_evaluation(length, dim):
    pin_tables_exact(length, dim)


@pytest.mark.parametrize("wk", [2, 3, 4, 5])
def test_workload_tables_sampled_exact(wk):
    w = workloads.WORKLOADS[wk]
    rng = np.random.Generator(np.random.PCG64(1234 + wk))
    for (T, H, W) in w.grids:
        for L, d in zip((T, H, W), w.split):
            ents = [(int(rng.integers(0, L)), int(rng.integers(0, d // 2))) for _ in range(12)]
            ents += [(L - 1, d // 2 - 1), (L - 1, 0)]
            pin_tables_exact(L, d, w.base, entries=ents)


def test_workload1_tables_exact():
    w = workloads.WORKLOADS[1]
    for L, d in zip(w.grids[0], w.split):
        pin_tables_exact(L, d, w.base)


@pytest.mark.parametrize("length,dim", [(17, 32), (120, 32), (96, 48), (6, 16)])
def test_table_closed_forms(length, dim):
    pin_table_closed_forms(length, dim)


def test_unit_vectors():
    pin_unit_vectors((2, 3, 4), (4, 8, 6))
    pin_unit_vectors((2, 4, 4), (16, 16, 16), heads=1)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_identity_at_origin(dtype):
    pin_identity_at_origin(dtype)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_zero_sections_unchanged(dtype):
    pin_zero_sections_unchanged(dtype)


def test_norm_preservation_and_round_trip():
    pin_norm_and_round_trip()


def test_complex_product_error_bound():
    pin_complex_product_bound()


def test_brute_force_workload1():
    w = workloads.WORKLOADS[1]
    (q, k), = workloads.generate(w)
    qo, ko = orc.rope3d_qk(q, k, w.dtype, w.split, w.base)
    bq, bk = _brute_force_qk(q, k, w.dtype, w.split, w.base)
    np.testing.assert_array_equal(qo.view(np.uint32), bq.view(np.uint32))
    np.testing.assert_array_equal(ko.view(np.uint32), bk.view(np.uint32))


@pytest.mark.parametrize("shape,dtype,split,seed", [
    ((1, 2, 3, 2, 2, 16), oracle.F32, (4, 8, 4), 21),
    ((2, 2, 2, 3, 1, 12), oracle.BF16, (4, 4, 4), 22),
    ((1, 5, 4, 3, 2, 20), oracle.BF16, (2, 6, 12), 23),
    ((2, 3, 1, 5, 3, 14), oracle.F32, (6, 2, 6), 24),
])
def test_brute_force_tiny_grids(shape, dtype, split, seed):
    pin_brute_force(shape, dtype, split, seed)


def test_sampled_equals_full():
    pin_sampled_equals_full()


@pytest.mark.parametrize("shape,dtype,split,offsets", [
    ((1, 2, 2, 3, 1, 12), oracle.BF16, (4, 4, 4), (3, 1, 2)),
    ((2, 1, 3, 2, 2, 16), oracle.F32, (4, 8, 4), (5, 0, 7)),
])
def test_brute_force_shards(shape, dtype, split, offsets):
    pin_brute_force(shape, dtype, split, 27, offsets=offsets)


def test_shard_is_slab_of_full():
    pin_shard_is_slab_of_full((2, 6, 5, 7, 2, 24), (8, 8, 8), (2, 1, 3), (3, 3, 4), 26)
    pin_shard_is_slab_of_full((1, 4, 4, 4, 3, 32), (8, 8, 16), (0, 2, 0), (4, 2, 4), 28)


def test_shard_outside_grid_rejected():
    q, k = workloads.generate_custom((1, 2, 2, 2, 1, 12), oracle.BF16, 1)
    with pytest.raises(ValueError):
        orc.rope3d(q, oracle.BF16, (4, 4, 4), offsets=(1, 0, 0), grid=(2, 2, 2))
    with pytest.raises(ValueError):
        orc.rope3d(q, oracle.BF16, (4, 4, 4), offsets=(-1, 0, 0))


def test_bf16_cast_against_torch_and_closed_forms():
    pin_bf16_cast()


def test_nan_results_are_canonical():
    pin_nan_canonical()


def test_validate_rejects_page_rules():
    with pytest.raises(ValueError):
        orc.validate((1, 2, 3, 4, 5), (2, 2, 2))
    with pytest.raises(ValueError):
        orc.validate((1, 2, 3, 4, 5, 6), (2, 2, 3))
    with pytest.raises(ValueError):
        orc.validate((1, 2, 3, 4, 5, 8), (2, 2, 2))
    with pytest.raises(ValueError):
        orc.validate((1, 0, 3, 4, 5, 6), (2, 2, 2))
    with pytest.raises(ValueError):
        orc.validate((1, 2, 3, 4, 5, 6), (0, 4, 2))


# ---------------------------------------------------------------------------
# planted mistakes: every one must be caught by at least one pin
# ---------------------------------------------------------------------------

def _rot_sign_flip(even, odd, cos, sin):
    f = np.float32
    return (np.add(np.multiply(even, cos, dtype=f), np.multiply(odd, sin, dtype=f), dtype=f),
            np.subtract(np.multiply(odd, cos, dtype=f), np.multiply(even, sin, dtype=f), dtype=f))


def _rot_swap_cs(even, odd, cos, sin):
    return orc.__dict__["_orig_rotate_pairs"](even, odd, sin, cos)


def _rot_drop_term(even, odd, cos, sin):
    f = np.float32
    return (np.multiply(even, cos, dtype=f),
            np.add(np.multiply(even, sin, dtype=f), np.multiply(odd, cos, dtype=f), dtype=f))


def _rot_fused(even, odd, cos, sin):
    e, o, c, s = (np.asarray(a, np.float64) for a in (even, odd, cos, sin))
    return (e * c - o * s).astype(np.float32), (e * s + o * c).astype(np.float32)


def _inv_freqs_wrong_exponent(dim, base):
    return [math.pow(base, -float(i) / dim) for i in range(dim // 2)]


def _token_coords_hw_swapped(token_ids, T, H, W):
    n = np.asarray(token_ids, dtype=np.int64) % (T * H * W)
    return n // (H * W), n % H, (n // H) % W


def _bf16_truncate(x):
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_ties_up(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)


def _apply_axis_order_swapped(x, dtype, coords, tables, split):
    t, h, w = coords
    return orc.__dict__["_orig_apply_rope_tokens"](x, dtype, (h, t, w), (tables[1], tables[0], tables[2]),
                                                   (split[1], split[0], split[2]))


def _apply_rotate_half(x, dtype, coords, tables, split):
    # NeoX rotate-half pairing (i, i + d/2) instead of interleaved (2i, 2i+1)
    M, heads, D = x.shape
    x32 = orc.to_f32(x, dtype)
    pieces, off = [], 0
    for d, (cos_a, sin_a), pos in zip(split, tables, coords):
        chunk = x32[:, :, off:off + d]
        even, odd = chunk[..., : d // 2], chunk[..., d // 2:]
        ye, yo = orc.rotate_pairs(even, odd, cos_a[pos][:, None, :], sin_a[pos][:, None, :])
        pieces.append(orc.from_f32(np.concatenate([ye, yo], axis=-1), dtype))
        off += d
    return np.concatenate(pieces, axis=-1)


def _axis_tables_off_by_one(length, dim, base):
    cos, sin = orc.__dict__["_orig_axis_tables"](length + 1, dim, base)
    return cos[1:].copy(), sin[1:].copy()


def _rope3d_offsets_ignored(x, dtype, split, base=10000.0, tables=None, offsets=(0, 0, 0), grid=None):
    B, T, H, W = x.shape[:4]
    g = grid if grid is not None else (T + offsets[0], H + offsets[1], W + offsets[2])
    if tables is None:
        tables = orc.grid_tables(*g, split, base)
    return orc.__dict__["_orig_rope3d"](x, dtype, split, base, tables, (0, 0, 0), g)


def _rope3d_offsets_rotated(x, dtype, split, base=10000.0, tables=None, offsets=(0, 0, 0), grid=None):
    t0, h0, w0 = offsets
    B, T, H, W = x.shape[:4]
    g = grid if grid is not None else (T + t0, H + h0, W + w0)
    return orc.__dict__["_orig_rope3d"](x, dtype, split, base, tables, (h0, w0, t0) if
                                        (h0 + T <= g[0] and w0 + H <= g[1] and t0 + W <= g[2]) else (0, 0, 0), g)


def _from_f32_keeps_nan_payload(y, dtype):
    if dtype == oracle.BF16:
        u = np.ascontiguousarray(y, dtype=np.float32).view(np.uint32).astype(np.uint64)
        return ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    return np.asarray(y, dtype=np.float32)


MUTATIONS = [
    ("rotate_pairs", _rot_sign_flip),
    ("rotate_pairs", _rot_swap_cs),
    ("rotate_pairs", _rot_drop_term),
    ("rotate_pairs", _rot_fused),
    ("inv_freqs", _inv_freqs_wrong_exponent),
    ("token_coords", _token_coords_hw_swapped),
    ("f32_to_bf16_bits", _bf16_truncate),
    ("f32_to_bf16_bits", _bf16_ties_up),
    ("apply_rope_tokens", _apply_axis_order_swapped),
    ("apply_rope_tokens", _apply_rotate_half),
    ("axis_tables", _axis_tables_off_by_one),
    ("rope3d", _rope3d_offsets_ignored),
    ("rope3d", _rope3d_offsets_rotated),
    ("from_f32", _from_f32_keeps_nan_payload),
]


@pytest.mark.parametrize("name,impl", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, impl):
    monkeypatch.setitem(orc.__dict__, "_orig_" + name, getattr(orc, name))
    monkeypatch.setattr(orc, name, impl)
    caught = []
    for pin_name, pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin_name)
    # the sampled path goes through token_coords; check it against the full path too
    try:
        pin_sampled_equals_full()
    except AssertionError:
        caught.append("sampled")
    assert caught, f"planted mistake {impl.__name__} in {name} passed every pin"
