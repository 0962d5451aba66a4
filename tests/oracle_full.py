"""Whole-tensor comparison of a GPU result with the oracle at full size (3D RoPE, rotate-half RoPE,
patchify).

For the 3D RoPE the oracle is applied one block of rows of one (batch, frame) at a time -- each block as a shard of
the whole grid, with the whole grid's tables -- from a pool of threads (numpy releases the
interpreter lock inside its array operations), and every element of the block is compared bit for
bit with the same block of the GPU output.  Blocks hold at most about 8 M elements, which bounds
the oracle's temporaries per thread.  Test helper only.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def pool_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32) if x.dtype == np.float32 else x.view(np.uint16)


BLOCK_ELEMS = 1 << 23


def compare_full(x_host: np.ndarray, got_host: np.ndarray, dtype: str, split, base: float, tables=None,
                 threads: int | None = None):
    """(mismatching elements, first mismatch or None) of got_host against the oracle on x_host,
    every element, 0 ULP (raw bits: NaN outputs are the canonical quiet NaN on both sides)."""
    B, T, H, W, heads, D = x_host.shape
    assert got_host.shape == x_host.shape and got_host.dtype == x_host.dtype
    if tables is None:
        tables = oracle.grid_tables(T, H, W, split, base)
    rows = max(1, min(H, BLOCK_ELEMS // (W * heads * D)))
    blocks = [(b, t, h0) for b in range(B) for t in range(T) for h0 in range(0, H, rows)]

    def block(job):
        b, t, h0 = job
        h1 = min(H, h0 + rows)
        x = np.ascontiguousarray(x_host[b:b + 1, t:t + 1, h0:h1])
        want = oracle.rope3d(x, dtype, split, base, tables=tables, offsets=(t, h0, 0), grid=(T, H, W))
        got = got_host[b:b + 1, t:t + 1, h0:h1]
        neq = bits(got) != bits(want)
        n = int(neq.sum())
        first = None
        if n:
            idx = tuple(int(v) for v in np.argwhere(neq)[0])
            loc = (b, t, h0 + idx[2]) + idx[3:]
            first = (loc, hex(int(bits(got)[idx])), hex(int(bits(want)[idx])))
        return n, first

    with ThreadPoolExecutor(threads or pool_threads()) as ex:
        results = list(ex.map(block, blocks))
    total = sum(n for n, _ in results)
    first = next((f for n, f in results if n), None)
    return total, first


def compare_full_neox(x_host: np.ndarray, got_host: np.ndarray, dtype: str, positions: np.ndarray,
                      cache: np.ndarray, cache_dtype: str, threads: int | None = None):
    """(mismatching elements, first mismatch or None) of got_host against oracle.neox on x_host
    ([tokens, heads, D]), every element, 0 ULP on raw bits.  The oracle runs over blocks of
    consecutive tokens (at most about 8 M elements each, every token with its own position's
    cache row) from a pool of threads."""
    import oracle.neox as nx

    tokens, heads, D = x_host.shape
    assert got_host.shape == x_host.shape and got_host.dtype == x_host.dtype
    step = max(1, BLOCK_ELEMS // (heads * D))

    def block(t0):
        t1 = min(tokens, t0 + step)
        want = nx.neox_rope(np.ascontiguousarray(x_host[t0:t1]), dtype, positions[t0:t1], cache, cache_dtype)
        got = got_host[t0:t1]
        neq = bits(got) != bits(want)
        n = int(neq.sum())
        first = None
        if n:
            idx = tuple(int(v) for v in np.argwhere(neq)[0])
            first = ((t0 + idx[0],) + idx[1:], hex(int(bits(got)[idx])), hex(int(bits(want)[idx])))
        return n, first

    with ThreadPoolExecutor(threads or pool_threads()) as ex:
        results = list(ex.map(block, range(0, tokens, step)))
    return sum(n for n, _ in results), next((f for n, f in results if n), None)


def compare_full_patchify(x_host: np.ndarray, y_host: np.ndarray, p: int, threads: int | None = None) -> int:
    """Elements of the patchified y_host that differ from oracle.patchify applied to x_host, over
    every (batch, channel, frame) plane, from a pool of threads."""
    import oracle.patchify as pf

    B, C, F, H, W = x_host.shape
    assert y_host.shape == (B, C * p * p, F, H // p, W // p) and y_host.dtype == x_host.dtype

    def plane(job):
        b, c, f = job
        want = pf.patchify(x_host[b:b + 1, c:c + 1, f:f + 1], p)[0, :, 0]
        return int((y_host[b, c * p * p:(c + 1) * p * p, f] != want).sum())

    jobs = [(b, c, f) for b in range(B) for c in range(C) for f in range(F)]
    with ThreadPoolExecutor(threads or pool_threads()) as ex:
        return sum(ex.map(plane, jobs))
