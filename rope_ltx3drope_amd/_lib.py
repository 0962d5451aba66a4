"""ctypes declarations of the ltx3drope C ABI (include/ltx3drope.h).

Loading fails loudly when the HIP library has not been built: there is no CPU
fallback anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libltx3drope.so")

OK = 0
E_INVALID = -1
E_UNSUPPORTED = -2
E_TABLE_MISMATCH = -3
E_HIP = -4
E_NOMEM = -5

DTYPE_F32 = 0
DTYPE_BF16 = 1

REASONS = {
    0: "OK", 1: "NULLPTR", 2: "DTYPE", 3: "NONPOSITIVE_DIM", 4: "SPLIT_ODD", 5: "SPLIT_SUM",
    6: "TABLE_GRID", 7: "TABLE_DEVICE", 8: "ALIGN", 9: "OVERLAP", 10: "TOO_LARGE",
    11: "NOT_DEVICE_PTR", 12: "HOST_MODE", 13: "EXTENT",
}
REASON_CODES = {v: k for k, v in REASONS.items()}

OPT_PATH = 1
OPT_GATE = 2
OPT_FORCE_GATE_MISMATCH = 3
OPT_HOST_TABLES = 4
OPT_LOG = 5

GATE_STATES = {0: "UNSEEN", 1: "TRUSTED", 2: "DISABLED"}

# every symbol the header declares (checked by the CPU test suite)
EXPORTS = (
    "ltx3drope_tables_build", "ltx3drope_tables_release", "ltx3drope_tables_describe", "ltx3drope_tables_read",
    "ltx3drope_cache_clear", "ltx3drope_can_use", "ltx3drope_apply_qk", "ltx3drope_apply_qk_noalloc",
    "ltx3drope_can_use_shard",
    "ltx3drope_apply_qk_shard", "ltx3drope_neox_can_use", "ltx3drope_neox_apply_qk",
    "ltx3drope_neox_position_errors", "ltx3drope_patchify", "ltx3drope_unpatchify", "ltx3drope_dit_freq_grid",
    "ltx3drope_gate_state",
    "ltx3drope_gate_reset", "ltx3drope_set_option", "ltx3drope_get_option", "ltx3drope_stats",
    "ltx3drope_stats_reset", "ltx3drope_kernel_choice", "ltx3drope_copy", "ltx3drope_status_string",
    "ltx3drope_reason_string", "ltx3drope_version",
)

i64 = ctypes.c_int64
vp = ctypes.c_void_p
fp = ctypes.POINTER(ctypes.c_float)


class TablesDesc(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int), ("T", i64), ("H", i64), ("W", i64), ("dim_t", i64), ("dim_h", i64),
                ("dim_w", i64), ("base", ctypes.c_double), ("packed", vp), ("packed_pairs", i64)]


class Shard(ctypes.Structure):
    _fields_ = [("t_offset", i64), ("h_offset", i64), ("w_offset", i64), ("inplace", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [(n, i64) for n in (
        "cache_hits", "cache_misses", "cache_evictions", "cache_live", "tables_alive", "gate_verifications",
        "gate_trusted", "gate_disabled", "fast_launches", "plain_launches", "rejected")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"ltx3drope HIP library not found at {LIB_PATH}; build it with "
                "`python -m rope_ltx3drope_amd.build` (there is no CPU fallback)")
        # torch first: its HIP runtime must be the process's one.  torch links the runtime under
        # another name than this library does, so loading this library first would bring in a
        # second runtime, to which torch's streams and allocations are unknown.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "ltx3drope_tables_build": (ctypes.c_int, [ctypes.c_int, i64, i64, i64, i64, i64, i64, ctypes.c_double, vp,
                                                      ctypes.POINTER(vp)]),
            "ltx3drope_tables_release": (ctypes.c_int, [vp]),
            "ltx3drope_tables_describe": (ctypes.c_int, [vp, ctypes.POINTER(TablesDesc)]),
            "ltx3drope_tables_read": (ctypes.c_int, [vp, fp, fp, fp, fp, fp, fp]),
            "ltx3drope_cache_clear": (ctypes.c_int, []),
            "ltx3drope_can_use": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64, vp,
                                                 ctypes.POINTER(ctypes.c_int)]),
            "ltx3drope_apply_qk": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64, vp, vp]),
            "ltx3drope_apply_qk_noalloc": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                                          vp, vp]),
            "ltx3drope_can_use_shard": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                                       ctypes.POINTER(Shard), vp, ctypes.POINTER(ctypes.c_int)]),
            "ltx3drope_apply_qk_shard": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                                        ctypes.POINTER(Shard), vp, vp]),
            "ltx3drope_neox_can_use": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, vp, vp,
                                                      ctypes.c_int, i64, ctypes.POINTER(ctypes.c_int)]),
            "ltx3drope_neox_apply_qk": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, vp, vp,
                                                       ctypes.c_int, i64, vp]),
            "ltx3drope_neox_position_errors": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.POINTER(i64)]),
            "ltx3drope_patchify": (ctypes.c_int, [vp, vp, ctypes.c_int] + [i64] * 6 + [vp]),
            "ltx3drope_unpatchify": (ctypes.c_int, [vp, vp, ctypes.c_int] + [i64] * 6 + [vp]),
            "ltx3drope_dit_freq_grid": (ctypes.c_int, [ctypes.c_double, i64, i64, ctypes.c_int, vp, vp,
                                                       ctypes.POINTER(i64)]),
            "ltx3drope_gate_state": (ctypes.c_int, [ctypes.c_int, ctypes.c_int] + [i64] * 9),
            "ltx3drope_gate_reset": (ctypes.c_int, []),
            "ltx3drope_set_option": (ctypes.c_int, [ctypes.c_int, i64]),
            "ltx3drope_get_option": (i64, [ctypes.c_int]),
            "ltx3drope_stats": (ctypes.c_int, [ctypes.POINTER(Stats)]),
            "ltx3drope_stats_reset": (ctypes.c_int, []),
            "ltx3drope_kernel_choice": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                                       vp]),
            "ltx3drope_copy": (ctypes.c_int, [vp, vp, i64, vp]),
            "ltx3drope_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "ltx3drope_reason_string": (ctypes.c_char_p, [ctypes.c_int]),
            "ltx3drope_version": (ctypes.c_int, []),
        }
        assert set(sig) == set(EXPORTS)
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
        return L


def status_string(code: int) -> str:
    return lib().ltx3drope_status_string(code).decode()


def reason_string(code: int) -> str:
    return lib().ltx3drope_reason_string(code).decode()
