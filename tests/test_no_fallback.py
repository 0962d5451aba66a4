"""CPU test: without the built HIP library every binding call raises; nothing falls back to a CPU
or torch computation."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import rope_ltx3drope_amd as rla
from rope_ltx3drope_amd import _lib
_lib.LIB_PATH = sys.argv[2]  # a library that does not exist
calls = {
    "tables_build": lambda: rla.tables_build(2, 2, 2, (2, 2, 2)),
    "neox_position_errors": rla.neox_position_errors,
    "cache_clear": rla.cache_clear,
    "dit_freq_grid": lambda: rla.dit_freq_grid(10000.0, 12, 6, True),
    "stats": rla.stats,
    "version": rla.version,
    "set_option": lambda: rla.set_option(rla.OPT_PATH, 0),
}
for name, call in calls.items():
    try:
        call()
    except RuntimeError as e:
        assert "no CPU fallback" in str(e), (name, e)
    except Exception as e:  # anything else would mean the call got past the library check
        raise SystemExit(f"{name}: {type(e).__name__}: {e}")
    else:
        raise SystemExit(f"{name}: returned without the library")
print("all refused")
"""


def test_every_entry_fails_loudly_without_the_library(tmp_path):
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT, str(tmp_path / "missing.so")], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all refused" in r.stdout
