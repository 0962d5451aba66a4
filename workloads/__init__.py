"""Seeded synthetic inputs for the fused 3D RoPE workloads.

This module holds the workload shapes and the random-number recipes only.
It contains none of the rotary arithmetic (no tables, no rotation, no
rounding of results), so both the CPU oracle and the GPU path can take
their inputs from it without sharing any of the method's code.

The decoder pages measure the RoPE on LTX-2.5 decoder tiles (stage 0/4/5)
whose exact geometries are not printed; the workloads below stand in for
them: Q/K shaped [B, T, H, W, heads, head_dim], contiguous, with token
n = (t*H + h)*W + w and the head dimension split into (dim_t, dim_h, dim_w)
channels (sglang PR #35698 page, "Key source snippets", JIT wrapper: the
six q dimensions and the per-axis table shapes of the precheck).

Representation: fp32 arrays are numpy float32; bf16 arrays are numpy
uint16 holding the raw bf16 bit patterns.  The fp32 -> bf16 conversion of
the drawn normals is done by torch's CPU cast (round to nearest even),
a library routine that neither the oracle nor the HIP path uses.
"""
from __future__ import annotations

import dataclasses
from typing import Iterator, List, Sequence, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload: a dtype, a batch/heads/head_dim shape and one or more grids."""

    key: int
    name: str
    dtype: str
    B: int
    grids: Tuple[Tuple[int, int, int], ...]
    heads: int
    head_dim: int
    split: Tuple[int, int, int]
    base: float
    seed: int
    dist: str  # "normal" or "normal3_outliers"
    calls: Tuple[int, ...]  # the order in which grids are visited (indices into grids)

    def shape(self, grid_index: int = 0) -> Tuple[int, int, int, int, int, int]:
        T, H, W = self.grids[grid_index]
        return (self.B, T, H, W, self.heads, self.head_dim)

    def numel(self, grid_index: int = 0) -> int:
        return int(np.prod(self.shape(grid_index), dtype=np.int64))

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == F32 else 2

    def algorithmic_bytes(self, grid_index: int = 0) -> int:
        """Q and K each read once and written once."""
        return 2 * 2 * self.numel(grid_index) * self.itemsize


WORKLOADS = {
    1: Workload(1, "tiny_f32_2x4x4_h2_d48", F32, 1, ((2, 4, 4),), 2, 48, (16, 16, 16),
                10000.0, 0, "normal", (0,)),
    2: Workload(2, "bf16_4x32x32_h16_d128", BF16, 1, ((4, 32, 32),), 16, 128, (32, 48, 48),
                10000.0, 1, "normal", (0,)),
    3: Workload(3, "stage4_tile_bf16_8x64x64_h24_d128_x24calls", BF16, 1, ((8, 64, 64),), 24, 128,
                (32, 48, 48), 10000.0, 2, "normal", (0,) * 24),
    4: Workload(4, "stage5_tile_bf16_16x96x96_h24_d128_outliers", BF16, 1, ((16, 96, 96),), 24, 128,
                (32, 48, 48), 10000.0, 3, "normal3_outliers", (0,)),
    5: Workload(5, "ragged_bf16_b2_17x68x120_h32_d96_3grids", BF16, 2,
                ((17, 68, 120), (9, 68, 120), (17, 34, 60)), 32, 96, (32, 32, 32),
                10000.0, 4, "normal", (0, 1, 2) * 4),
}

_CHUNK = 1 << 24  # elements drawn per numpy call; the stream is sequential so chunking is invisible


def _f32_to_bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    import torch  # CPU only; used as a library cast for input generation

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _draw_normal(rng: np.random.Generator, n: int, dtype: str, scale: float | None) -> np.ndarray:
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if scale is not None:
            v = np.multiply(v, np.float32(scale), dtype=np.float32)
        out[s:e] = v if dtype == F32 else _f32_to_bf16_bits_torch(v)
    return out


def _outlier_value_bits(value: float, dtype: str):
    if dtype == F32:
        return np.float32(value)
    return _f32_to_bf16_bits_torch(np.array([value], dtype=np.float32))[0]


def generate(w: Workload, grid_indices: Sequence[int] | None = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Return [(q, k), ...] for the requested grids, drawn from one generator.

    One numpy PCG64 generator seeded with the workload's seed draws, in
    order and in C order: for each grid of the workload, all of Q then all
    of K.  Grids before the last requested one are still drawn (to keep
    the stream order) but dropped.  For "normal3_outliers" the values are 3*N(0,1) (an fp32
    multiply before the cast), then for Q and then K about 0.1 % of the
    flat positions (rng.integers, duplicates allowed) are set to +60 or -60
    with the sign drawn by rng.integers(0, 2).
    """
    want = set(range(len(w.grids))) if grid_indices is None else set(grid_indices)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    out = []
    for gi in range(max(want) + 1):
        n = w.numel(gi)
        scale = 3.0 if w.dist == "normal3_outliers" else None
        q = _draw_normal(rng, n, w.dtype, scale)
        k = _draw_normal(rng, n, w.dtype, scale)
        if w.dist == "normal3_outliers":
            pos = _outlier_value_bits(60.0, w.dtype)
            neg = _outlier_value_bits(-60.0, w.dtype)
            for x in (q, k):
                cnt = int(round(1e-3 * n))
                idx = rng.integers(0, n, size=cnt)
                sign = rng.integers(0, 2, size=cnt)
                x[idx] = np.where(sign == 1, pos, neg).astype(x.dtype)
        if gi in want:
            shp = w.shape(gi)
            out.append((q.reshape(shp), k.reshape(shp)))
    return out


def generate_bf16_bits(shape: Sequence[int], seed: int, device):
    """Finite bf16 bit patterns of random sign and mantissa with magnitudes in [1/8, 2), drawn with
    torch's seeded generator on `device` (a torch bf16 tensor): for the largest tensors, billions
    of elements, which are generated where they are used rather than on the host."""
    import torch

    g = torch.Generator(device=device).manual_seed(seed)
    raw = torch.empty(tuple(shape), dtype=torch.int16, device=device).random_(-32768, 32768, generator=g)
    raw.bitwise_and_(-32257).bitwise_or_(0x3E00)  # keep sign and mantissa (0x81FF); exponent field 0x7C..0x7F
    return raw.view(torch.bfloat16)


def generate_neox_device(tokens: int, q_heads: int, k_heads: int, head_dim: int, max_position: int, seed: int,
                         device):
    """Rotate-half RoPE inputs of any size drawn with torch's seeded generator on `device`: q, k
    bf16 tensors of N(0,1) values (torch's fp32 draw and cast) and int64 positions uniform in
    [0, max_position).  For token counts whose host generation would take minutes."""
    import torch

    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn(tokens, q_heads, head_dim, generator=g, device=device).to(torch.bfloat16)
    k = torch.randn(tokens, k_heads, head_dim, generator=g, device=device).to(torch.bfloat16)
    pos = torch.randint(0, max_position, (tokens,), generator=g, device=device, dtype=torch.int64)
    return q, k, pos


def generate_custom(shape: Sequence[int], dtype: str, seed: int, scale: float | None = None):
    """Q, K of an arbitrary [B,T,H,W,heads,D] shape with N(0,1)*scale values (tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape, dtype=np.int64))
    q = _draw_normal(rng, n, dtype, scale).reshape(shape)
    k = _draw_normal(rng, n, dtype, scale).reshape(shape)
    return q, k


def sample_tokens(num_tokens: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct flat token indices (b*N + n) used for sampled comparisons."""
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    count = min(count, num_tokens)
    idx = rng.choice(num_tokens, size=count, replace=False)
    # always include the first and last token so both ends of the tensor are checked
    idx = np.unique(np.concatenate([idx, [0, num_tokens - 1]]))
    return idx.astype(np.int64)


def iter_calls(w: Workload) -> Iterator[int]:
    yield from w.calls


# ---------------------------------------------------------------------------
# rotate-half RoPE with a gathered cos/sin cache (text-encoder rotary)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class NeoxWorkload:
    """q [tokens, q_heads, D], k [tokens, k_heads, D], positions [tokens], cache [max_position, D]."""

    key: str
    dtype: str
    tokens: int
    q_heads: int
    k_heads: int
    head_dim: int
    max_position: int
    cache_dtype: str
    positions: str  # "arange" (a prefill) or "random"
    seed: int

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == F32 else 2

    def algorithmic_bytes(self) -> int:
        """Q and K read once and written once, the positions read once, one cache row read per token."""
        qk = (self.q_heads + self.k_heads) * self.head_dim * self.itemsize
        cache_row = self.head_dim * (4 if self.cache_dtype == F32 else 2)
        return self.tokens * (2 * qk + 8 + cache_row)


NEOX_WORKLOADS = {
    "n1": NeoxWorkload("n1_f32_tiny", F32, 7, 4, 2, 16, 32, F32, "random", 10),
    "n2": NeoxWorkload("n2_bf16_prefill_1k", BF16, 1024, 16, 8, 256, 4096, F32, "arange", 11),
    "n3": NeoxWorkload("n3_bf16_random_pos", BF16, 3000, 8, 4, 128, 8192, BF16, "random", 12),
    "n4": NeoxWorkload("n4_bf16_32k_tokens_h16_kv8_d256", BF16, 32768, 16, 8, 256, 32768, F32, "arange", 13),
}


def generate_neox(w: NeoxWorkload):
    """(q, k, positions, cache).  The cache rows are cos|sin of angles drawn uniformly in
    [-pi, pi) (float64 numpy cos/sin, rounded to the cache dtype by torch's cast): the op under
    test only gathers and consumes them, so any unit-circle values are representative."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    n_q = w.tokens * w.q_heads * w.head_dim
    n_k = w.tokens * w.k_heads * w.head_dim
    q = _draw_normal(rng, n_q, w.dtype, None).reshape(w.tokens, w.q_heads, w.head_dim)
    k = _draw_normal(rng, n_k, w.dtype, None).reshape(w.tokens, w.k_heads, w.head_dim)
    if w.positions == "arange":
        pos = np.arange(w.tokens, dtype=np.int64) % w.max_position
    else:
        pos = rng.integers(0, w.max_position, size=w.tokens, dtype=np.int64)
    ang = rng.uniform(-np.pi, np.pi, size=(w.max_position, w.head_dim // 2))
    rows = np.concatenate([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    cache = rows if w.cache_dtype == F32 else _f32_to_bf16_bits_torch(rows.reshape(-1)).reshape(rows.shape)
    return q, k, pos, cache


# ---------------------------------------------------------------------------
# stage-5 space-to-depth (patchify) inputs: (B, C, F, H, W) tensors of raw bits
# ---------------------------------------------------------------------------

PATCH_WORKLOADS = {
    # key: (shape (B, C, F, H, W), p, element bytes)
    "p1": ((1, 3, 5, 16, 24), 4, 4),        # W not a multiple of p*4 -> plain kernel
    "p2": ((1, 3, 9, 64, 96), 4, 2),
    "p3": ((2, 16, 5, 32, 48), 2, 2),
    "p4": ((1, 3, 3, 64, 128), 8, 2),
    "p5": ((1, 4, 7, 40, 80), 4, 4),
    "p6": ((1, 3, 121, 544, 960), 4, 2),     # every frame of a 121 x 544 x 960 RGB clip, bf16
    "p7": ((1, 2, 3, 6, 48), 2, 2),          # bf16, p = 2, last wavefront partly filled
    "p8": ((1, 3, 5, 8, 40), 2, 4),          # fp32, p = 2, last wavefront partly filled
    "p9": ((1, 2, 3, 16, 64), 8, 4),         # fp32, p = 8: a vector does not split across 8 offsets
    "p10": ((1, 1, 3, 24, 192), 8, 2),       # bf16, p = 8, last wavefront partly filled
    "p11": ((1, 5, 1, 4, 64), 4, 2),         # bf16, p = 4, one partly filled wavefront
    "p12": ((1, 3, 121, 544, 960), 8, 4),    # the 121-frame clip in fp32 with p = 8
    # element sizes and patch sizes where a vector's elements and p divide one another either way
    "p13": ((1, 3, 3, 6, 64), 2, 1),          # u8, p = 2
    "p14": ((1, 1, 5, 4, 128), 4, 1),         # u8, p = 4, one partly filled workgroup
    "p15": ((1, 3, 2, 32, 256), 16, 1),       # u8, p = 16: 16-wavefront workgroups
    "p16": ((1, 1, 2, 32, 256), 16, 2),       # bf16, p = 16
    "p17": ((1, 3, 5, 16, 96), 8, 4),         # fp32, p = 8: each element to its own plane
    "p18": ((1, 1, 2, 32, 128), 16, 4),       # fp32, p = 16
    "p19": ((1, 3, 3, 6, 20), 2, 8),          # 8-byte elements, p = 2
    "p20": ((2, 3, 3, 16, 48), 8, 8),         # 8-byte elements, p = 8, partly filled
    "p21": ((1, 3, 3, 16, 64), 16, 8),        # 8-byte elements, p = 16
}


def generate_patch_device(shape, elem_bytes: int, seed: int, device):
    """Random bit patterns of the element width drawn with torch's seeded generator on `device`
    (a torch integer tensor of that width), for tensors too large to draw on the host quickly."""
    import torch

    dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[elem_bytes]
    g = torch.Generator(device=device).manual_seed(seed)
    lo, hi = (0, 256) if elem_bytes == 1 else (-(1 << (8 * elem_bytes - 1)), 1 << (8 * elem_bytes - 1))
    if elem_bytes == 8:
        lo, hi = -(1 << 62), 1 << 62  # random_ wants both bounds representable
    return torch.empty(tuple(shape), dtype=dt, device=device).random_(lo, hi, generator=g)


def generate_patch(shape, elem_bytes: int, seed: int) -> np.ndarray:
    """Random bit patterns of the element width (the op moves data without reading values)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[elem_bytes]
    return rng.integers(0, np.iinfo(dt).max, size=shape, dtype=dt, endpoint=True)
