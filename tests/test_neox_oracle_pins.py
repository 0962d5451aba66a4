"""Pins of the rotate-half RoPE oracle (oracle.neox) against independent references.

* fp32: the rotate-half rotation of (x[i], x[i + D/2]) is the interleaved pair
  rotation of the 3D oracle (itself pinned against mathematics) applied to the
  de-interleaved layout, with the cache halves as the (cos, sin) table.
* bf16 and fp32: the page's expression executed by torch on the CPU (torch's
  own dtype rules: every op computes in fp32 and rounds to the tensor dtype).
* closed forms: identity where cos = 1 and sin = 0, unit vectors, an error
  bound against the exact rotation, and planted mistakes that must be caught.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.neox as nx
import oracle.rope as orc
import workloads


def _inputs(tokens=9, heads=3, D=16, max_pos=20, dtype=oracle.BF16, cache_dtype=oracle.F32, seed=1):
    w = workloads.NeoxWorkload("t", dtype, tokens, heads, 1, D, max_pos, cache_dtype, "random", seed)
    q, _, pos, cache = workloads.generate_neox(w)
    return q, pos, cache


def _torch_dtype(d):
    return torch.bfloat16 if d == oracle.BF16 else torch.float32


def _to_torch(x, d):
    if d == oracle.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x))


def _from_torch(t, d):
    if d == oracle.BF16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def torch_page_expression(q, dtype, pos, cache, cache_dtype):
    """The page's expression, evaluated by torch on the CPU."""
    qt = _to_torch(q, dtype)
    ct = _to_torch(cache, cache_dtype)
    cos_sin = ct.index_select(0, torch.from_numpy(pos))
    cos, sin = cos_sin.chunk(2, dim=-1)
    cos = torch.cat((cos, cos), dim=-1).to(dtype=qt.dtype).unsqueeze(1)
    sin = torch.cat((sin, sin), dim=-1).to(dtype=qt.dtype).unsqueeze(1)
    d = qt.shape[-1] // 2
    rh = torch.cat((-qt[..., d:], qt[..., :d]), dim=-1)
    return _from_torch(qt * cos + rh * sin, dtype)


def bits(x):
    return x.view(np.uint32) if x.dtype == np.float32 else x.view(np.uint16)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_fp32_equals_interleaved_3d_oracle(seed=3):
    q, pos, cache = _inputs(dtype=oracle.F32, seed=seed, tokens=11, heads=2, D=24, max_pos=30)
    D = q.shape[-1]
    got = nx.neox_rope(q, oracle.F32, pos, cache, oracle.F32)
    # interleave (x[i], x[i + D/2]) into pairs, rotate with the 3D oracle's pair rotation
    inter = np.stack([q[..., : D // 2], q[..., D // 2:]], axis=-1).reshape(q.shape)
    table = (cache[:, : D // 2].copy(), cache[:, D // 2:].copy())
    rot = orc.apply_rope_tokens(inter, oracle.F32, (pos,), (table,), (D,))
    rot = rot.reshape(q.shape[0], q.shape[1], D // 2, 2)
    want = np.concatenate([rot[..., 0], rot[..., 1]], axis=-1)
    np.testing.assert_array_equal(bits(got), bits(want))


def pin_torch_expression(dtype, cache_dtype, seed=4):
    q, pos, cache = _inputs(dtype=dtype, cache_dtype=cache_dtype, seed=seed, tokens=33, heads=4, D=32, max_pos=64)
    got = nx.neox_rope(q, dtype, pos, cache, cache_dtype)
    want = torch_page_expression(q, dtype, pos, cache, cache_dtype)
    np.testing.assert_array_equal(bits(got), bits(want))


def pin_identity_and_unit_vectors():
    D = 8
    cache = np.zeros((3, D), np.float32)
    cache[0, : D // 2] = 1.0                     # position 0: cos 1, sin 0
    ang = np.array([0.3, -1.1, 2.0, 0.7])
    cache[1, : D // 2], cache[1, D // 2:] = np.cos(ang), np.sin(ang)
    cache[2] = cache[1]
    x = workloads.generate_custom((1, 1, 1, 1, 4, D), oracle.F32, 5)[0].reshape(4, 1, D)
    y = nx.neox_rope(x, oracle.F32, np.zeros(4, np.int64), cache, oracle.F32)
    np.testing.assert_array_equal(y, x)
    eye = np.eye(D, dtype=np.float32).reshape(D, 1, D)
    y = nx.neox_rope(eye, oracle.F32, np.ones(D, np.int64), cache, oracle.F32)
    c, s = cache[1, : D // 2], cache[1, D // 2:]
    for i in range(D // 2):
        # e_i -> c_i at i, s_i at i + D/2 ; e_{i+D/2} -> -s_i at i, c_i at i + D/2
        assert y[i, 0, i] == c[i] and y[i, 0, i + D // 2] == s[i]
        assert y[i + D // 2, 0, i] == -s[i] and y[i + D // 2, 0, i + D // 2] == c[i]
        assert np.count_nonzero(y[i, 0]) == 2 and np.count_nonzero(y[i + D // 2, 0]) == 2


def pin_error_bound(dtype=oracle.BF16, seed=6):
    q, pos, cache = _inputs(dtype=dtype, seed=seed, tokens=40, heads=3, D=32, max_pos=50)
    D = q.shape[-1]
    got = oracle.to_f32(nx.neox_rope(q, dtype, pos, cache, oracle.F32), dtype).astype(np.float64)
    cs = oracle.to_f32(oracle.from_f32(cache[pos], dtype), dtype).astype(np.float64)[:, None, :]
    x = oracle.to_f32(q, dtype).astype(np.float64)
    c, s = cs[..., : D // 2], cs[..., D // 2:]
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    exact = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    mag = np.concatenate([np.abs(x1 * c) + np.abs(x2 * s), np.abs(x2 * c) + np.abs(x1 * s)], axis=-1)
    u = 2.0 ** -8 if dtype == oracle.BF16 else 2.0 ** -24  # unit roundoff of the dtype
    assert np.all(np.abs(got - exact) <= mag * 2 * u + np.abs(exact) * 2 * u + 1e-30)


def pin_nan_canonical():
    """A NaN result is the canonical quiet NaN whatever the sign and payload of the NaN input."""
    for dtype, nans, canon in ((oracle.F32, np.array([0xFFC00000, 0x7F800001, 0xFF812345], np.uint32).view(np.float32),
                                0x7FC00000),
                               (oracle.BF16, np.array([0xFFC0, 0x7F81, 0xFF92], np.uint16), 0x7FC0)):
        q, pos, cache = _inputs(tokens=4, heads=2, D=8, dtype=dtype, seed=12)
        q.reshape(-1)[[0, 5, 9]] = nans
        out = nx.neox_rope(q, dtype, pos, cache, oracle.F32)
        raw = out.view(np.uint32) if dtype == oracle.F32 else out
        nan = np.isnan(oracle.to_f32(out, dtype))
        assert nan.sum() >= 3 and np.all(raw[nan] == canon)


ALL_PINS = [
    ("fp32_vs_3d", pin_fp32_equals_interleaved_3d_oracle),
    ("torch_bf16_f32cache", lambda: pin_torch_expression(oracle.BF16, oracle.F32)),
    ("torch_bf16_bf16cache", lambda: pin_torch_expression(oracle.BF16, oracle.BF16)),
    ("torch_f32", lambda: pin_torch_expression(oracle.F32, oracle.F32)),
    ("closed_forms", pin_identity_and_unit_vectors),
    ("bound_bf16", pin_error_bound),
    ("nan_canonical", pin_nan_canonical),
]


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(name, pin):
    pin()


def test_torch_expression_many_seeds_and_shapes():
    for seed, (tokens, heads, D, max_pos) in enumerate([(5, 1, 2, 3), (17, 8, 64, 100), (64, 2, 256, 80)]):
        for dtype, cdt in ((oracle.BF16, oracle.F32), (oracle.BF16, oracle.BF16), (oracle.F32, oracle.F32),
                           (oracle.F32, oracle.BF16)):
            q, pos, cache = _inputs(tokens, heads, D, max_pos, dtype, cdt, seed=40 + seed)
            np.testing.assert_array_equal(bits(nx.neox_rope(q, dtype, pos, cache, cdt)),
                                          bits(torch_page_expression(q, dtype, pos, cache, cdt)))


def test_rejects_bad_positions_and_shapes():
    q, pos, cache = _inputs()
    with pytest.raises(ValueError):
        nx.neox_rope(q, oracle.BF16, pos + 100, cache, oracle.F32)
    with pytest.raises(ValueError):
        nx.neox_rope(q, oracle.BF16, -pos - 1, cache, oracle.F32)
    with pytest.raises(ValueError):
        nx.neox_rope(q[..., :15], oracle.BF16, pos, cache, oracle.F32)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _rh_wrong_sign(x):
    d = x.shape[-1] // 2
    return np.concatenate([x[..., d:], -x[..., :d]], axis=-1)


def _rh_interleaved(x):
    y = np.empty_like(x)
    y[..., 0::2] = -x[..., 1::2]
    y[..., 1::2] = x[..., 0::2]
    return y


def _round_to_skip_bf16(x32, dtype):
    return np.asarray(x32, dtype=np.float32)  # never rounds to bf16 between ops


def _neox_positions_ignored(x, dtype, positions, cache, cache_dtype):
    return nx.__dict__["_orig_neox_rope"](x, dtype, np.arange(x.shape[0]) % cache.shape[0], cache, cache_dtype)


def _neox_cos_sin_swapped(x, dtype, positions, cache, cache_dtype):
    D = cache.shape[-1]
    sw = np.concatenate([cache[:, D // 2:], cache[:, : D // 2]], axis=-1)
    return nx.__dict__["_orig_neox_rope"](x, dtype, positions, sw, cache_dtype)


def _neox_keeps_nan_payload(x, dtype, positions, cache, cache_dtype):
    y = nx.__dict__["_orig_neox_rope"](x, dtype, positions, cache, cache_dtype)
    if dtype != oracle.F32:
        return y
    xf = np.asarray(x, np.float32)
    out = y.copy()
    nan = np.isnan(out) & np.isnan(xf)
    out[nan] = xf[nan]  # the input's NaN pattern instead of the canonical one
    return out


MUTATIONS = [
    ("rotate_half", _rh_wrong_sign),
    ("rotate_half", _rh_interleaved),
    ("round_to", _round_to_skip_bf16),
    ("neox_rope", _neox_positions_ignored),
    ("neox_rope", _neox_cos_sin_swapped),
    ("neox_rope", _neox_keeps_nan_payload),
]


@pytest.mark.parametrize("name,impl", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, impl):
    monkeypatch.setitem(nx.__dict__, "_orig_" + name, getattr(nx, name))
    monkeypatch.setattr(nx, name, impl)
    caught = []
    for pin_name, pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"planted mistake {impl.__name__} in {name} passed every pin"
