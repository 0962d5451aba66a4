"""CPU checks of the full-size comparison helpers (tests/oracle_full.py) that the GPU parity tests
rely on: run over many small blocks, they agree with one whole-tensor application of the oracle,
and they find and locate a single changed element."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.neox as nx
import workloads
from tests import oracle_full


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.F32])
def test_compare_full_blocks_agree_with_the_whole_tensor(monkeypatch, dtype):
    shape, split, base = (2, 3, 5, 7, 3, 24), (8, 8, 8), 10000.0
    x, _ = workloads.generate_custom(shape, dtype, seed=5)
    whole = oracle.rope3d(x, dtype, split, base)
    # blocks of two rows of one (batch, frame): 3 blocks per frame, the last one ragged
    monkeypatch.setattr(oracle_full, "BLOCK_ELEMS", 2 * 7 * 3 * 24)
    assert oracle_full.compare_full(x, whole, dtype, split, base, threads=3) == (0, None)
    bad = whole.copy()
    loc = (1, 2, 4, 6, 2, 17)
    oracle_full.bits(bad)[loc] ^= 1  # flip the lowest bit of one element
    n, first = oracle_full.compare_full(x, bad, dtype, split, base, threads=3)
    assert n == 1 and first[0] == loc


def test_compare_full_catches_a_wrong_block_offset(monkeypatch):
    """A result computed with the rows' table offset lost (every block rotated as if it started at
    row 0) must not pass: the helper takes each block's offsets from its place in the grid."""
    shape, split, base = (1, 2, 6, 4, 2, 12), (4, 4, 4), 10000.0
    x, _ = workloads.generate_custom(shape, oracle.BF16, seed=6)
    wrong = np.concatenate([oracle.rope3d(np.ascontiguousarray(x[:, :, h0:h0 + 2]), oracle.BF16, split, base)
                            for h0 in range(0, 6, 2)], axis=2)
    monkeypatch.setattr(oracle_full, "BLOCK_ELEMS", 2 * 4 * 2 * 12)
    n, _ = oracle_full.compare_full(x, wrong, oracle.BF16, split, base, threads=2)
    assert n > 0


@pytest.mark.parametrize("key", ["n1", "n3"])
def test_compare_full_neox_blocks_agree_with_the_whole_tensor(monkeypatch, key):
    w = workloads.NEOX_WORKLOADS[key]
    q, k, pos, cache = workloads.generate_neox(w)
    monkeypatch.setattr(oracle_full, "BLOCK_ELEMS", 5 * w.q_heads * w.head_dim)  # 5 tokens per block
    for x in (q, k):
        whole = nx.neox_rope(x, w.dtype, pos, cache, w.cache_dtype)
        assert oracle_full.compare_full_neox(x, whole, w.dtype, pos, cache, w.cache_dtype, threads=3) == (0, None)
        bad = whole.copy()
        loc = (x.shape[0] - 1, x.shape[1] - 1, 3)
        oracle_full.bits(bad)[loc] ^= 1
        n, first = oracle_full.compare_full_neox(x, bad, w.dtype, pos, cache, w.cache_dtype, threads=3)
        assert n == 1 and first[0] == loc


def test_compare_full_neox_catches_positions_shifted_by_a_block():
    """Every token must meet its own position's cache row: a result whose positions were taken
    from the wrong tokens fails."""
    w = workloads.NEOX_WORKLOADS["n3"]
    q, _, pos, cache = workloads.generate_neox(w)
    wrong = nx.neox_rope(q, w.dtype, np.roll(pos, 5), cache, w.cache_dtype)
    n, _ = oracle_full.compare_full_neox(q, wrong, w.dtype, pos, cache, w.cache_dtype, threads=2)
    assert n > 0


def test_compare_full_patchify_planes_agree_with_the_whole_tensor():
    import oracle.patchify as pf

    x = workloads.generate_patch((2, 3, 4, 8, 12), 2, seed=3)
    y = pf.patchify(x, 4)
    assert oracle_full.compare_full_patchify(x, y, 4, threads=3) == 0
    bad = y.copy()
    bad[1, 2 * 16 + 5, 3, 1, 2] ^= 1
    assert oracle_full.compare_full_patchify(x, bad, 4, threads=3) == 1
    # the channel packing order matters: height and width offsets swapped must fail
    swapped = x.reshape(2, 3, 4, 2, 4, 3, 4).transpose(0, 1, 4, 6, 2, 3, 5).reshape(2, 48, 4, 2, 3)
    assert oracle_full.compare_full_patchify(x, np.ascontiguousarray(swapped), 4, threads=3) > 0
