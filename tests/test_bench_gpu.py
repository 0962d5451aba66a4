"""bench.py's JSON line on the GPU: every op prints one line with the contract's fields, parity 0."""
from __future__ import annotations

import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

rla = pytest.importorskip("rope_ltx3drope_amd")

CONTRACT = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def run_bench(capsys, monkeypatch, *argv):
    monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    return json.loads(lines[0])


@pytest.mark.parametrize("argv", [
    ("--workload", "2", "--steps", "3", "--warmup", "2", "--no-cpu-baseline"),
    ("--workload", "1", "--steps", "3", "--warmup", "2", "--graph", "--no-cpu-baseline"),
    ("--workload", "2", "--steps", "2", "--warmup", "1", "--inplace", "--no-cpu-baseline"),
    ("--op", "neox", "--neox-workload", "n2", "--steps", "3", "--warmup", "2", "--no-cpu-baseline"),
    ("--op", "patchify", "--patch-workload", "p2", "--steps", "3", "--warmup", "2", "--no-cpu-baseline"),
    ("--op", "unpatchify", "--patch-workload", "p2", "--steps", "3", "--warmup", "2", "--no-cpu-baseline"),
    ("--op", "dit_freqs", "--steps", "3", "--warmup", "2"),
    ("--workload", "3", "--cycle", "--steps", "2", "--warmup", "1"),
], ids=["rope3d", "rope3d-graph", "rope3d-inplace", "neox", "patchify", "unpatchify", "dit", "rope3d-cycle"])
def test_bench_line(capsys, monkeypatch, argv):
    rla.set_option(rla.OPT_PATH, 0)
    d = run_bench(capsys, monkeypatch, *argv)
    assert CONTRACT <= set(d), CONTRACT - set(d)
    assert d["n_gpus"] == 1 and d["value"] > 0 and d["steps"] == int(argv[argv.index("--steps") + 1])
    assert d["parity"]["mismatching_elements"] == 0
    assert "workload" in d["config"]
    if "timed_region_device_allocations" in d:  # outputs are reserved before the warmup
        assert d["timed_region_device_allocations"] == 0
    if d["roofline"] is not None:
        r = d["roofline"]
        assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
        assert 0 < r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-3)


def test_cycle_mode_reports_the_table_cache(capsys, monkeypatch):
    """Workload 3's 24 calls as one step: one table build in the warmup, hits ever after."""
    rla.set_option(rla.OPT_PATH, 0)
    d = run_bench(capsys, monkeypatch, "--workload", "3", "--cycle", "--steps", "2", "--warmup", "1")
    assert d["config"]["call_sequence"] == [0] * 24
    assert d["table_cache"] == {"warmup_misses": 1, "warmup_hits": 23, "timed_misses": 0, "timed_hits": 48}
    assert d["kernel"] == "rope_fast" and d["parity"]["mismatching_elements"] == 0
