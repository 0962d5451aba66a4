"""Plain CPU oracle for the fused LTX-2.5 decoder 3D rotary position embedding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, links or
calls this module; only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the benchmark do.  It shares no code, table or
constant generator with the HIP path.

What it computes (sglang PR #35698 page, "Implementation breakdown", steps 1
and 2, and "Key source snippets", the CUDA kernel snippet):

* Per-axis tables.  For an axis of length L and rotary width d (an even
  number of channels), the table holds cos and sin of the angle
  theta(p, i) = p * base**(-2 i / d) for integer positions p in [0, L) and
  pair columns i in [0, d/2).  The page names the builder (_axis_tables) but
  does not print its formula; this is the textbook inverse-frequency RoPE
  that the builder replaced (_inv_freqs), with integer positions because the
  cache key carries no offset or scale.  Computed in float64 (Python's math
  module) and rounded once to fp32.  Whether sglang's own tables hold the
  same bits cannot be checked: no table values are printed anywhere.

* The eager rotation.  The head dimension is cut into a time, a height and a
  width chunk of (dim_t, dim_h, dim_w) channels, in that order.  Each chunk
  is viewed as interleaved (even, odd) pairs; in fp32, with every product and
  sum rounded separately (no fused multiply-add), the pair becomes
      even*cos - odd*sin ,  even*sin + odd*cos
  using the table row of the token's t, h or w coordinate; the result is cast
  back to the input dtype (round to nearest even for bf16) and the three
  chunks are concatenated again.  Q and K use the same tables.

Representation: fp32 tensors are numpy float32 arrays; bf16 tensors are numpy
uint16 arrays of raw bf16 bits.  Layout [B, T, H, W, heads, D], token
n = (t*H + h)*W + w.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"

Tables = Tuple[Tuple[np.ndarray, np.ndarray], Tuple[np.ndarray, np.ndarray], Tuple[np.ndarray, np.ndarray]]


# ---------------------------------------------------------------------------
# tables (sglang PR #35698 page, "Implementation breakdown", step 1)
# ---------------------------------------------------------------------------

def inv_freqs(dim: int, base: float) -> list:
    """omega_i = base ** (-(2 i) / dim) for i in [0, dim/2), in float64."""
    return [math.pow(base, -(2.0 * i) / dim) for i in range(dim // 2)]


def axis_tables(length: int, dim: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    """(cos, sin) of one axis as fp32 arrays of shape [length, dim/2].

    The angle is one float64 product of the position and omega_i; cos and
    sin are evaluated in float64 and rounded once to fp32 (numpy's
    double -> float conversion rounds to nearest even).
    """
    om = inv_freqs(dim, base)
    cos = np.empty((length, dim // 2), dtype=np.float32)
    sin = np.empty((length, dim // 2), dtype=np.float32)
    for p in range(length):
        for i, w in enumerate(om):
            theta = float(p) * w
            cos[p, i] = math.cos(theta)
            sin[p, i] = math.sin(theta)
    return cos, sin


def grid_tables(T: int, H: int, W: int, split: Sequence[int], base: float = 10000.0) -> Tables:
    """The three (cos, sin) pairs for a (T, H, W) grid, in t, h, w order."""
    dim_t, dim_h, dim_w = split
    return (axis_tables(T, dim_t, base), axis_tables(H, dim_h, base), axis_tables(W, dim_w, base))


# ---------------------------------------------------------------------------
# dtype conversions
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: the bf16 bits become the top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); any NaN becomes 0x7FC0.

    Adding 0x7FFF plus the lowest kept bit to the fp32 pattern and dropping
    the low 16 bits rounds to nearest with ties going to the even neighbour;
    overflow past the largest finite bf16 carries into the infinity pattern.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, np.uint16(0x7FC0), rounded).astype(np.uint16)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == BF16 else np.asarray(x, dtype=np.float32)


def f32_canonical_nan(y: np.ndarray) -> np.ndarray:
    """fp32 values with every NaN replaced by the canonical quiet NaN 0x7FC00000 (the pages are
    silent on NaN payloads; one fixed pattern makes equal inputs give byte-identical outputs)."""
    y = np.asarray(y, dtype=np.float32)
    nan = np.isnan(y)
    if not nan.any():
        return y
    out = y.copy()
    out.view(np.uint32)[nan] = np.uint32(0x7FC00000)
    return out


def from_f32(y: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(y) if dtype == BF16 else f32_canonical_nan(y)


# ---------------------------------------------------------------------------
# rotation (sglang PR #35698 page, "Implementation breakdown", step 2, and the
# pair-rotation helper of the CUDA kernel snippet under "Key source snippets")
# ---------------------------------------------------------------------------

def rotate_pairs(even: np.ndarray, odd: np.ndarray, cos: np.ndarray, sin: np.ndarray):
    """fp32 rotation of (even, odd) by the angle whose cos/sin are given.

    Four products, each rounded to fp32, then one rounded difference and one
    rounded sum.  Separate numpy ufunc calls cannot fuse into an FMA.
    """
    f = np.float32
    with np.errstate(over="ignore", invalid="ignore"):
        t1 = np.multiply(even, cos, dtype=f)  # e c
        t2 = np.multiply(odd, sin, dtype=f)   # o s
        t3 = np.multiply(even, sin, dtype=f)  # e s
        t4 = np.multiply(odd, cos, dtype=f)   # o c
        return np.subtract(t1, t2, dtype=f), np.add(t3, t4, dtype=f)


def validate(shape: Sequence[int], split: Sequence[int]) -> None:
    """The shape rules of the page's precheck (JIT wrapper snippet, can_use)."""
    if len(shape) != 6:
        raise ValueError("expected a 6-D [B, T, H, W, heads, D] tensor")
    if any(int(s) <= 0 for s in shape):
        raise ValueError("all sizes must be positive")
    if len(split) != 3 or any(d <= 0 or d % 2 for d in split):
        raise ValueError("rope_dim_split must be three positive even numbers")
    if shape[-1] != sum(split):
        raise ValueError("head_dim must equal dim_t + dim_h + dim_w")


def apply_rope_tokens(x: np.ndarray, dtype: str, coords: Sequence[np.ndarray], tables: Tables,
                      split: Sequence[int]) -> np.ndarray:
    """The eager rotation of M tokens: x is [M, heads, D]; coords = (t, h, w), each [M].

    For each axis chunk of the head dimension (t, h, w in order): view the
    chunk as (even, odd) pairs, rotate in fp32 with that axis's table row at
    the token's coordinate, cast back to the input dtype; then concatenate
    the chunks along the head dimension.
    """
    M, heads, D = x.shape
    x32 = to_f32(x, dtype)
    pieces = []
    off = 0
    for d, (cos_a, sin_a), pos in zip(split, tables, coords):
        chunk = x32[:, :, off:off + d].reshape(M, heads, d // 2, 2)
        even = chunk[..., 0]
        odd = chunk[..., 1]
        c = cos_a[pos][:, None, :]
        s = sin_a[pos][:, None, :]
        y_even, y_odd = rotate_pairs(even, odd, c, s)
        y = np.stack([y_even, y_odd], axis=-1).reshape(M, heads, d)
        pieces.append(from_f32(y, dtype))
        off += d
    return np.concatenate(pieces, axis=-1)


def token_coords(token_ids: np.ndarray, T: int, H: int, W: int):
    """Flat token index (b*T*H*W + n) -> (t, h, w) with n = (t*H + h)*W + w."""
    n = np.asarray(token_ids, dtype=np.int64) % (T * H * W)
    return n // (H * W), (n // W) % H, n % W


def rope3d(x: np.ndarray, dtype: str, split: Sequence[int], base: float = 10000.0,
           tables: Tables | None = None, offsets: Sequence[int] = (0, 0, 0),
           grid: Sequence[int] | None = None) -> np.ndarray:
    """Rotate one [B, T, H, W, heads, D] tensor; returns a new array of the same dtype.

    offsets / grid: the tensor may be a shard of a larger (T_g, H_g, W_g) grid
    (the frames, rows and columns [offset, offset + size) of each axis); a
    token then takes the table rows of its global coordinate, i.e. its local
    coordinate plus the axis offset.  By default the tensor is the whole grid.

    Processed one (b, t) slab at a time to bound host memory; every slab is
    an independent application of apply_rope_tokens.
    """
    validate(x.shape, split)
    B, T, H, W, heads, D = x.shape
    t0, h0, w0 = (int(o) for o in offsets)
    Tg, Hg, Wg = grid if grid is not None else (T + t0, H + h0, W + w0)
    if min(t0, h0, w0) < 0 or t0 + T > Tg or h0 + H > Hg or w0 + W > Wg:
        raise ValueError("the shard does not lie inside the grid")
    if tables is None:
        tables = grid_tables(Tg, Hg, Wg, split, base)
    out = np.empty_like(x)
    hh, ww = np.meshgrid(np.arange(H) + h0, np.arange(W) + w0, indexing="ij")
    hh = hh.reshape(-1)
    ww = ww.reshape(-1)
    for b in range(B):
        for t in range(T):
            tt = np.full(H * W, t + t0, dtype=np.int64)
            slab = x[b, t].reshape(H * W, heads, D)
            out[b, t] = apply_rope_tokens(slab, dtype, (tt, hh, ww), tables, split).reshape(H, W, heads, D)
    return out


def rope3d_qk(q: np.ndarray, k: np.ndarray, dtype: str, split: Sequence[int], base: float = 10000.0,
              tables: Tables | None = None, offsets: Sequence[int] = (0, 0, 0),
              grid: Sequence[int] | None = None):
    """(q_out, k_out): both tensors rotated with one shared table set."""
    if q.shape != k.shape:
        raise ValueError("q and k must have the same shape")
    validate(q.shape, split)
    B, T, H, W, heads, D = q.shape
    if grid is None:
        grid = (T + offsets[0], H + offsets[1], W + offsets[2])
    if tables is None:
        tables = grid_tables(*grid, split, base)
    return (rope3d(q, dtype, split, base, tables, offsets, grid),
            rope3d(k, dtype, split, base, tables, offsets, grid))


def rope3d_sampled(x: np.ndarray, dtype: str, split: Sequence[int], token_ids: np.ndarray,
                   base: float = 10000.0, tables: Tables | None = None, offsets: Sequence[int] = (0, 0, 0),
                   grid: Sequence[int] | None = None) -> np.ndarray:
    """Rotated rows [len(token_ids), heads, D] for selected flat token indices of x
    (x may be a shard of a larger grid, as in rope3d)."""
    validate(x.shape, split)
    B, T, H, W, heads, D = x.shape
    if grid is None:
        grid = (T + offsets[0], H + offsets[1], W + offsets[2])
    if tables is None:
        tables = grid_tables(*grid, split, base)
    ids = np.asarray(token_ids, dtype=np.int64)
    rows = x.reshape(B * T * H * W, heads, D)[ids]
    t, h, w = token_coords(ids, T, H, W)
    coords = (t + offsets[0], h + offsets[1], w + offsets[2])
    return apply_rope_tokens(rows, dtype, coords, tables, split)
