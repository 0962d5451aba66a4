"""rope_ltx3drope_amd: fused 3D RoPE of the LTX-2.5 diffusion video decoder on MI355X.

Thin Python binding of the ltx3drope C ABI (include/ltx3drope.h).  Every step
of the operation -- table construction and caching, the precheck, the gate and
the rotation kernels -- runs in the native library; this module only marshals
arguments.  PyTorch supplies device memory (torch.empty_like for the fresh
outputs, as the page's wrapper does) and the current HIP stream.  If the
library is missing, every call raises: there is no CPU fallback.

Names follow the sglang PR #35698 page ("Implementation breakdown", steps 1-4;
"Key source snippets"): tables() is the cached per-axis table lookup,
can_use() the precheck, apply_qk() the fused one-launch rotation of Q and K and
forward_pair() the decoder-side entry that ties them together.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

from . import _lib
from ._lib import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    GATE_STATES,
    OPT_FORCE_GATE_MISMATCH,
    OPT_GATE,
    OPT_HOST_TABLES,
    OPT_LOG,
    OPT_PATH,
    REASON_CODES,
    REASONS,
)

__all__ = [
    "Ltx3dRopeError", "Ltx3dRopeUnsupported", "Tables", "tables", "tables_build", "can_use", "apply_qk",
    "apply_qk_noalloc",
    "forward_pair", "kernel_choice", "stats", "stats_reset", "set_option", "get_option", "gate_state", "gate_reset",
    "cache_clear", "copy_bytes", "version", "neox_can_use", "neox_apply_qk", "neox_position_errors", "patchify",
    "unpatchify", "dit_freq_grid",
]


class Ltx3dRopeError(RuntimeError):
    """A library call failed (status code in .status)."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.status_string(status)} ({status})")
        self.status = status


class Ltx3dRopeUnsupported(Ltx3dRopeError):
    """The precheck rejected the inputs; nothing was launched (reason name in .reason)."""

    def __init__(self, reason: str, status: int = _lib.E_UNSUPPORTED):
        RuntimeError.__init__(self, f"unsupported input: {reason}")
        self.status = status
        self.reason = reason


def _check(status: int, what: str) -> None:
    if status != _lib.OK:
        raise Ltx3dRopeError(status, what)


def _refused(status: int, reason: ctypes.c_int, what: str):
    """The error for an apply call that the library refused: the precheck's reason, or, where the
    precheck passes, the library's refusal of host-memory tables (host-table test mode)."""
    if reason.value == 0:
        return Ltx3dRopeUnsupported("HOST_MODE" if get_option(OPT_HOST_TABLES) else f"{what}: refused", status)
    return Ltx3dRopeUnsupported(_lib.REASONS.get(reason.value, str(reason.value)), status)


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    return -1


def _stream_ptr(device, stream=None) -> int:
    """The hipStream_t of `stream`, or of torch's current stream on `device` (a torch device or an
    index)."""
    torch = _torch()
    if stream is not None:
        return int(stream.cuda_stream)
    idx = device if isinstance(device, int) else device.index
    if idx is None:
        idx = torch.cuda.current_device()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)  # the same pointer, without a Stream object
    if raw is not None:
        return int(raw(idx))
    return int(torch.cuda.current_stream(idx).cuda_stream)


class Tables:
    """A reference to one cached table set (released on close() / garbage collection)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("tables already released")
        return self._h

    def describe(self) -> dict:
        d = _lib.TablesDesc()
        _check(_lib.lib().ltx3drope_tables_describe(self.handle, ctypes.byref(d)), "tables_describe")
        return {"device": d.device, "grid": (d.T, d.H, d.W), "split": (d.dim_t, d.dim_h, d.dim_w), "base": d.base,
                "packed": d.packed, "packed_pairs": d.packed_pairs}

    @property
    def grid(self) -> Tuple[int, int, int]:
        return self.describe()["grid"]

    @property
    def split(self) -> Tuple[int, int, int]:
        return self.describe()["split"]

    def read(self):
        """The six tables as numpy fp32 arrays ((cos_t, sin_t), (cos_h, sin_h), (cos_w, sin_w))."""
        import numpy as np

        d = self.describe()
        shapes = [(L, dd // 2) for L, dd in zip(d["grid"], d["split"])]
        arrs = [np.empty(s, np.float32) for s in shapes for _ in range(2)]
        ptrs = [a.ctypes.data_as(_lib.fp) for a in arrs]
        _check(_lib.lib().ltx3drope_tables_read(self.handle, *ptrs), "tables_read")
        return (arrs[0], arrs[1]), (arrs[2], arrs[3]), (arrs[4], arrs[5])

    def close(self) -> None:
        if self._h:
            _lib.lib().ltx3drope_tables_release(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def tables_build(T: int, H: int, W: int, split: Sequence[int], base: float = 10000.0, device: int = 0,
                 stream=None) -> Tables:
    """Find or build the per-axis tables of a (T, H, W) grid (FIFO cache of 16 entries)."""
    dt, dh, dw = (int(x) for x in split)
    out = ctypes.c_void_p()
    host_mode = get_option(OPT_HOST_TABLES) != 0
    sp = 0 if host_mode else _stream_ptr(int(device), stream)
    _check(_lib.lib().ltx3drope_tables_build(int(device), int(T), int(H), int(W), dt, dh, dw, float(base), sp,
                                              ctypes.byref(out)), "tables_build")
    return Tables(out.value)


tables = tables_build


def _shape6(q):
    if q.dim() != 6:
        raise Ltx3dRopeUnsupported("NOT_6D")
    return tuple(int(s) for s in q.shape)


def _marshal(q, k, q_out, k_out):
    if k.shape != q.shape:
        raise Ltx3dRopeUnsupported("SHAPE_MISMATCH")
    if k.dtype != q.dtype:
        raise Ltx3dRopeUnsupported("DTYPE")
    if not (q.is_cuda and k.is_cuda) or q.device != k.device:
        raise Ltx3dRopeUnsupported("NOT_DEVICE_PTR")
    for t in (q, k, q_out, k_out):
        if t is not None and not t.is_contiguous():
            raise Ltx3dRopeUnsupported("NOT_CONTIGUOUS")
    for t in (q_out, k_out):
        if t is not None and (t.shape != q.shape or t.dtype != q.dtype or t.device != q.device):
            raise Ltx3dRopeUnsupported("OUTPUT_MISMATCH")


def _shard(offsets, inplace):
    """A shard descriptor, or None for the unsharded, out-of-place entry points."""
    if offsets is None and not inplace:
        return None
    t0, h0, w0 = (int(x) for x in (offsets or (0, 0, 0)))
    return _lib.Shard(t0, h0, w0, 1 if inplace else 0, 0)


def can_use(q, k, tabs: Tables, q_out=None, k_out=None, offsets=None, inplace: bool = False) -> Tuple[bool, str]:
    """The precheck: (True, "OK") if apply_qk would launch, else (False, reason).

    offsets: (t, h, w) position of q's first frame/row/column in the tables' grid (a shard);
    inplace: allow q_out is q and k_out is k."""
    try:
        B, T, H, W, heads, D = _shape6(q)
        _marshal(q, k, q_out, k_out)
    except Ltx3dRopeUnsupported as e:
        return False, e.reason
    qo = q_out.data_ptr() if q_out is not None else None
    ko = k_out.data_ptr() if k_out is not None else None
    if (qo is None) != (ko is None):
        raise ValueError("give both q_out and k_out, or neither")
    reason = ctypes.c_int(0)
    sh = _shard(offsets, inplace)
    if sh is None:
        ok = _lib.lib().ltx3drope_can_use(qo, ko, q.data_ptr(), k.data_ptr(), _dtype_code(q), B, T, H, W, heads, D,
                                          tabs.handle, ctypes.byref(reason))
    else:
        ok = _lib.lib().ltx3drope_can_use_shard(qo, ko, q.data_ptr(), k.data_ptr(), _dtype_code(q), B, T, H, W, heads,
                                                D, ctypes.byref(sh), tabs.handle, ctypes.byref(reason))
    return bool(ok), _lib.REASONS.get(reason.value, str(reason.value))


def apply_qk(q, k, tabs: Tables, q_out=None, k_out=None, stream=None, offsets=None, inplace: bool = False):
    """Rotate Q and K into fresh (or the given) output tensors with one kernel launch.

    offsets: (t, h, w) position of q's first frame/row/column in the tables' grid, for a shard of a
    larger grid; inplace=True rotates q and k in place (q_out/k_out must then be None or q/k)."""
    torch = _torch()
    B, T, H, W, heads, D = _shape6(q)
    _marshal(q, k, q_out, k_out)
    if inplace:
        if (q_out is not None and q_out is not q) or (k_out is not None and k_out is not k):
            raise ValueError("inplace=True writes into q and k")
        q_out, k_out = q, k
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    sh = _shard(offsets, inplace)
    args = (q_out.data_ptr(), k_out.data_ptr(), q.data_ptr(), k.data_ptr(), _dtype_code(q), B, T, H, W, heads, D)
    if sh is None:
        st = _lib.lib().ltx3drope_apply_qk(*args, tabs.handle, _stream_ptr(q.device, stream))
    else:
        st = _lib.lib().ltx3drope_apply_qk_shard(*args, ctypes.byref(sh), tabs.handle, _stream_ptr(q.device, stream))
    if st in (_lib.E_UNSUPPORTED, _lib.E_TABLE_MISMATCH):
        reason = ctypes.c_int(0)
        if sh is None:
            _lib.lib().ltx3drope_can_use(*args, tabs.handle, ctypes.byref(reason))
        else:
            _lib.lib().ltx3drope_can_use_shard(*args, ctypes.byref(sh), tabs.handle, ctypes.byref(reason))
        raise _refused(st, reason, "apply_qk")
    _check(st, "apply_qk")
    return q_out, k_out


def apply_qk_noalloc(q, k, tabs: Tables, q_out, k_out, stream=None):
    """apply_qk into caller-provided outputs through the entry point that allocates no device memory
    (the gate's verification counter is a static device array of the library)."""
    B, T, H, W, heads, D = _shape6(q)
    if q_out is None or k_out is None:
        raise ValueError("apply_qk_noalloc writes into caller-provided q_out and k_out")
    _marshal(q, k, q_out, k_out)
    args = (q_out.data_ptr(), k_out.data_ptr(), q.data_ptr(), k.data_ptr(), _dtype_code(q), B, T, H, W, heads, D)
    st = _lib.lib().ltx3drope_apply_qk_noalloc(*args, tabs.handle, _stream_ptr(q.device, stream))
    if st in (_lib.E_UNSUPPORTED, _lib.E_TABLE_MISMATCH):
        reason = ctypes.c_int(0)
        _lib.lib().ltx3drope_can_use(*args, tabs.handle, ctypes.byref(reason))
        raise _refused(st, reason, "apply_qk_noalloc")
    _check(st, "apply_qk_noalloc")
    return q_out, k_out


def forward_pair(q, k, split: Sequence[int], base: float = 10000.0, q_out=None, k_out=None, stream=None,
                 grid: Optional[Sequence[int]] = None, offsets=None, inplace: bool = False):
    """Decoder-side entry: cached tables for the grid, then the fused rotation.

    grid defaults to q's own (T, H, W) (plus offsets, for a shard at the end of its grid)."""
    B, T, H, W, heads, D = _shape6(q)
    if grid is None:
        t0, h0, w0 = offsets or (0, 0, 0)
        grid = (T + t0, H + h0, W + w0)
    if not q.is_cuda:
        raise Ltx3dRopeUnsupported("NOT_DEVICE_PTR")
    device = q.device.index if q.device.index is not None else _torch().cuda.current_device()
    with tables_build(*grid, split, base, device=device, stream=stream) as tabs:
        return apply_qk(q, k, tabs, q_out, k_out, stream, offsets, inplace)


def _neox_marshal(q, k, positions, cache, q_out, k_out):
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise Ltx3dRopeUnsupported("SHAPE_MISMATCH")
    if k.dtype != q.dtype or positions.dtype != torch.int64:
        raise Ltx3dRopeUnsupported("DTYPE")
    if positions.numel() != q.shape[0] or cache.dim() != 2 or cache.shape[1] != q.shape[2]:
        raise Ltx3dRopeUnsupported("SHAPE_MISMATCH")
    for t in (q, k, positions, cache):
        if not t.is_cuda or t.device != q.device:
            raise Ltx3dRopeUnsupported("NOT_DEVICE_PTR")
    for t in (q, k, positions, cache, q_out, k_out):
        if t is not None and not t.is_contiguous():
            raise Ltx3dRopeUnsupported("NOT_CONTIGUOUS")
    for t, ref in ((q_out, q), (k_out, k)):
        if t is not None and (t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device):
            raise Ltx3dRopeUnsupported("OUTPUT_MISMATCH")


def _neox_args(q_out, k_out, q, k, positions, cache):
    return (q_out.data_ptr() if q_out is not None else None, k_out.data_ptr() if k_out is not None else None,
            q.data_ptr(), k.data_ptr(), _dtype_code(q), int(q.shape[0]), int(q.shape[1]), int(k.shape[1]),
            int(q.shape[2]), positions.data_ptr(), cache.data_ptr(), _dtype_code(cache), int(cache.shape[0]))


def neox_can_use(q, k, positions, cache, q_out=None, k_out=None) -> Tuple[bool, str]:
    """Precheck of the rotate-half RoPE: q [tokens, q_heads, D], k [tokens, k_heads, D],
    positions [tokens] int64, cache [max_position, D] (cos half, then sin half)."""
    try:
        _neox_marshal(q, k, positions, cache, q_out, k_out)
    except Ltx3dRopeUnsupported as e:
        return False, e.reason
    if (q_out is None) != (k_out is None):
        raise ValueError("give both q_out and k_out, or neither")
    reason = ctypes.c_int(0)
    ok = _lib.lib().ltx3drope_neox_can_use(*_neox_args(q_out, k_out, q, k, positions, cache), ctypes.byref(reason))
    return bool(ok), _lib.REASONS.get(reason.value, str(reason.value))


def neox_apply_qk(q, k, positions, cache, q_out=None, k_out=None, inplace: bool = False, stream=None):
    """Rotate-half RoPE of Q and K with the cache rows gathered at `positions`, one launch."""
    torch = _torch()
    _neox_marshal(q, k, positions, cache, q_out, k_out)
    if inplace:
        if (q_out is not None and q_out is not q) or (k_out is not None and k_out is not k):
            raise ValueError("inplace=True writes into q and k")
        q_out, k_out = q, k
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    args = _neox_args(q_out, k_out, q, k, positions, cache)
    st = _lib.lib().ltx3drope_neox_apply_qk(*args, _stream_ptr(q.device, stream))
    if st == _lib.E_UNSUPPORTED:
        reason = ctypes.c_int(0)
        _lib.lib().ltx3drope_neox_can_use(*args, ctypes.byref(reason))
        raise Ltx3dRopeUnsupported(_lib.REASONS.get(reason.value, str(reason.value)), st)
    _check(st, "neox_apply_qk")
    return q_out, k_out


def neox_position_errors(device: int = 0, reset: bool = False) -> int:
    """(token, tensor) pairs whose position was outside the cache since the last reset (synchronizes)."""
    n = ctypes.c_int64(0)
    _check(_lib.lib().ltx3drope_neox_position_errors(int(device), 1 if reset else 0, ctypes.byref(n)),
           "neox_position_errors")
    return int(n.value)


def patchify(x, p: int, out=None, stream=None):
    """Space-to-depth (B, C, F, H, W) -> (B, C*p*p, F, H/p, W/p), channels packed as
    (channel, width offset, height offset)."""
    torch = _torch()
    if x.dim() != 5 or not x.is_cuda or not x.is_contiguous():
        raise Ltx3dRopeUnsupported("SHAPE_MISMATCH")
    B, C, F, H, W = (int(s) for s in x.shape)
    if p < 1 or H % p or W % p:
        raise ValueError("H and W must be multiples of p")
    shape = (B, C * p * p, F, H // p, W // p)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise Ltx3dRopeUnsupported("OUTPUT_MISMATCH")
    st = _lib.lib().ltx3drope_patchify(out.data_ptr(), x.data_ptr(), x.element_size(), B, C, F, H, W, int(p),
                                      _stream_ptr(x.device, stream))
    if st == _lib.E_UNSUPPORTED:
        raise Ltx3dRopeUnsupported("PRECHECK", st)
    _check(st, "patchify")
    return out


def unpatchify(y, p: int, out=None, stream=None):
    """Inverse of patchify: (B, C*p*p, F, H/p, W/p) -> (B, C, F, H, W)."""
    torch = _torch()
    if p < 1:
        raise ValueError("p must be positive")
    if y.dim() != 5 or not y.is_cuda or not y.is_contiguous() or int(y.shape[1]) % (p * p):
        raise Ltx3dRopeUnsupported("SHAPE_MISMATCH")
    B, Cpp, F, Hp, Wp = (int(s) for s in y.shape)
    C, H, W = Cpp // (p * p), Hp * p, Wp * p
    if out is None:
        out = torch.empty((B, C, F, H, W), dtype=y.dtype, device=y.device)
    elif tuple(out.shape) != (B, C, F, H, W) or out.dtype != y.dtype or not out.is_contiguous() or out.device != y.device:
        raise Ltx3dRopeUnsupported("OUTPUT_MISMATCH")
    st = _lib.lib().ltx3drope_unpatchify(out.data_ptr(), y.data_ptr(), y.element_size(), B, C, F, H, W, int(p),
                                        _stream_ptr(y.device, stream))
    if st == _lib.E_UNSUPPORTED:
        raise Ltx3dRopeUnsupported("PRECHECK", st)
    _check(st, "unpatchify")
    return out


def dit_freq_grid(theta: float, dim: int, num_rope_elems: int, double_precision: bool, device=None, stream=None):
    """LTX DiT RoPE frequencies (float32, dim // num_rope_elems values), generated by one kernel on
    `device` (a torch device; default: the current one) and returned as a device tensor."""
    L = _lib.lib()  # fails loudly when the library is missing, before any device is touched
    torch = _torch()
    if int(num_rope_elems) <= 0:
        raise ValueError("num_rope_elems must be positive")
    count = max(0, int(dim) // int(num_rope_elems))
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(count, dtype=torch.float32, device=device)
    if not out.is_cuda:
        raise Ltx3dRopeUnsupported("NOT_DEVICE_PTR")
    n = ctypes.c_int64(0)
    st = L.ltx3drope_dit_freq_grid(float(theta), int(dim), int(num_rope_elems), int(bool(double_precision)),
                                   out.data_ptr() if count else None, _stream_ptr(out.device, stream), ctypes.byref(n))
    if st == _lib.E_UNSUPPORTED:
        raise Ltx3dRopeUnsupported("NOT_DEVICE_PTR", st)
    _check(st, "dit_freq_grid")
    return out


def kernel_choice(q, k, tabs: Tables, q_out=None, k_out=None) -> str:
    """'fast' or 'plain': the kernel apply_qk uses once the gate trusts the fast path."""
    B, T, H, W, heads, D = _shape6(q)
    if (q_out is None) != (k_out is None):
        raise ValueError("give both q_out and k_out, or neither")
    qo = q_out.data_ptr() if q_out is not None else None
    ko = k_out.data_ptr() if k_out is not None else None
    r = _lib.lib().ltx3drope_kernel_choice(qo, ko, q.data_ptr(), k.data_ptr(), _dtype_code(q), B, T, H, W, heads, D,
                                           tabs.handle)
    if r < 0:
        raise Ltx3dRopeError(r, "kernel_choice")
    return {1: "fast", 2: "plain"}[r]


def stats() -> dict:
    s = _lib.Stats()
    _check(_lib.lib().ltx3drope_stats(ctypes.byref(s)), "stats")
    return s.as_dict()


def stats_reset() -> None:
    _check(_lib.lib().ltx3drope_stats_reset(), "stats_reset")


def set_option(option: int, value: int) -> None:
    _check(_lib.lib().ltx3drope_set_option(int(option), int(value)), "set_option")


def get_option(option: int) -> int:
    return int(_lib.lib().ltx3drope_get_option(int(option)))


def gate_state(device: int, dtype: int, shape: Sequence[int], split: Sequence[int]) -> str:
    r = _lib.lib().ltx3drope_gate_state(int(device), int(dtype), *[int(s) for s in shape], *[int(s) for s in split])
    if r < 0:
        raise Ltx3dRopeError(r, "gate_state")
    return GATE_STATES[r]


def gate_reset() -> None:
    _check(_lib.lib().ltx3drope_gate_reset(), "gate_reset")


def cache_clear() -> None:
    _check(_lib.lib().ltx3drope_cache_clear(), "cache_clear")


def copy_bytes(dst, src, nbytes: Optional[int] = None, stream=None) -> None:
    """Plain streaming copy kernel (bandwidth and counter calibration)."""
    n = int(nbytes if nbytes is not None else src.numel() * src.element_size())
    _check(_lib.lib().ltx3drope_copy(dst.data_ptr(), src.data_ptr(), n, _stream_ptr(src.device, stream)), "copy")


def version() -> int:
    return int(_lib.lib().ltx3drope_version())
