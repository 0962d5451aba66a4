"""Plain CPU oracle for the NeoX ("rotate-half") RoPE with a position-gathered cos/sin cache.

TEST INFRASTRUCTURE ONLY (like oracle.rope): only tests/, the graft entry
point's smoke check and bench.py's CPU baseline may use it.

What it computes (sglang PR #24660 page, "Key source snippets", the Gemma3
text encoder's rotary application; "Implementation breakdown", step 2: the
encoder looks its cos/sin up in a precomputed cache with index_select):

    cos_sin  = cache[positions]                 # gather one row per token
    cos, sin = cos_sin split into two halves    # [tokens, D/2] each
    cos      = concat(cos, cos) in q's dtype    # duplicated to the full head
    sin      = concat(sin, sin) in q's dtype
    q'       = q * cos + rotate_half(q) * sin   # the same for k
    rotate_half(x) = concat(-x[D/2:], x[:D/2])  # the usual rotate-half layout

Every tensor operation of that expression produces a tensor of q's dtype: the
products and the sum are computed in fp32 and rounded once to q's dtype (for
bf16, round to nearest even; for fp32, the fp32 rounding itself).  The cache
may be fp32 or bf16; the gathered values are converted to q's dtype first.

A NaN result is written as the canonical quiet NaN (0x7FC00000 in fp32, 0x7FC0
in bf16), as in oracle.rope: the page says nothing about NaN payloads.

Layout: q [tokens, q_heads, D], k [tokens, k_heads, D] (the head counts may
differ), positions [tokens] integers in [0, max_position), cache
[max_position, D] with the cos half first.  bf16 arrays are uint16 bit
patterns, fp32 arrays float32.
"""
from __future__ import annotations

import numpy as np

from .rope import BF16, F32, f32_canonical_nan, f32_to_bf16_bits, to_f32


def round_to(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the tensor dtype and return them as fp32 again."""
    if dtype == BF16:
        return to_f32(f32_to_bf16_bits(x32), BF16)
    return np.asarray(x32, dtype=np.float32)


def rotate_half(x: np.ndarray) -> np.ndarray:
    d = x.shape[-1] // 2
    return np.concatenate([-x[..., d:], x[..., :d]], axis=-1)


def neox_rope(x: np.ndarray, dtype: str, positions: np.ndarray, cache: np.ndarray, cache_dtype: str) -> np.ndarray:
    """x: [tokens, heads, D] -> rotated, same dtype and shape."""
    tokens, heads, D = x.shape
    if D % 2 or cache.shape[-1] != D:
        raise ValueError("head_dim must be even and equal to the cache row width")
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    if pos.shape[0] != tokens or pos.min(initial=0) < 0 or pos.max(initial=0) >= cache.shape[0]:
        raise ValueError("one position per token, inside the cache")
    rows = to_f32(np.asarray(cache)[pos], cache_dtype)         # index_select
    cos, sin = rows[:, : D // 2], rows[:, D // 2:]              # chunk(2, dim=-1)
    cos = round_to(np.concatenate([cos, cos], axis=-1), dtype)  # cat + .to(q.dtype)
    sin = round_to(np.concatenate([sin, sin], axis=-1), dtype)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    xf = to_f32(x, dtype)
    f = np.float32
    with np.errstate(over="ignore", invalid="ignore"):
        a = round_to(np.multiply(xf, cos, dtype=f), dtype)                # q * cos
        b = round_to(np.multiply(rotate_half(xf), sin, dtype=f), dtype)   # rotate_half(q) * sin
        y = round_to(np.add(a, b, dtype=f), dtype)                        # sum
    return f32_to_bf16_bits(y) if dtype == BF16 else f32_canonical_nan(y)


def neox_rope_qk(q, k, dtype, positions, cache, cache_dtype):
    """(q', k') with one shared gather of the cache."""
    return (neox_rope(q, dtype, positions, cache, cache_dtype),
            neox_rope(k, dtype, positions, cache, cache_dtype))
