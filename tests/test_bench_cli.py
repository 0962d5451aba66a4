"""bench.py's command line (CPU): the one-GPU rule, per-op defaults and argument checks."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import pytest  # noqa: E402

import bench  # noqa: E402


def parse(*argv):
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        return bench.parse()
    finally:
        sys.argv = old


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_defaults_per_op():
    a = parse()
    assert (a.op, a.workload, a.steps, a.warmup, a.gpus) == ("rope3d", 5, 50, 20, 1)
    for op in ("neox", "patchify", "unpatchify", "dit_freqs"):
        a = parse("--op", op)
        assert (a.steps, a.warmup) == (200, 200)
    a = parse("--steps", "7", "--warmup", "3")
    assert (a.steps, a.warmup) == (7, 3)


def test_head_share_and_cpu_thread_options():
    a = parse("--heads", "3")
    assert a.heads == 3
    assert 1 <= parse().cpu_threads <= 16
    assert parse("--cpu-threads", "0").cpu_threads == 0


def test_bad_step_counts_are_refused():
    for argv in (("--steps", "0"), ("--warmup", "-1"), ("--rotate", "-2")):
        with pytest.raises(SystemExit) as e:
            parse(*argv)
        assert e.value.code == 2


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a comment\nint x = 1;  // trailing\n/* block\ncomment */\nint y = 2;\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": ("k.hip",)})
    h1 = bench.kernel_source_hash("k")
    src.write_text("int x = 1;\n\n// other words\nint y = 2;\n")
    assert bench.kernel_source_hash("k") == h1
    src.write_text("int x = 1;\nint y = 3;\n")
    assert bench.kernel_source_hash("k") != h1


def test_every_timed_kernel_hashes_its_own_sources():
    for kernel, files in bench.KERNEL_SOURCES.items():
        assert all(os.path.exists(os.path.join(bench.CSRC, f)) for f in files), kernel
    assert bench.kernel_source_hash("patch_lds") == bench.kernel_source_hash("unpatch_lds")
    assert bench.kernel_source_hash("rope_fast") != bench.kernel_source_hash("neox_fast")


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_traffic_record_is_used_only_for_the_source_it_was_taken_on(kernel):
    """bench.py reports a kernel's committed counter traffic only for the workload and the kernel
    source the counters were taken on (else null)."""
    import json

    path = bench.traffic_file(kernel)
    if not os.path.exists(path):
        assert bench.measured_traffic("any", kernel) is None
        return
    rec = json.load(open(path))
    assert rec["kernel"] == kernel
    assert 1.0 <= rec["traffic_over_algorithmic"] < 1.05
    assert bench.measured_traffic("another workload", kernel) is None
    if rec["kernel_source_sha256_16"] == bench.kernel_source_hash(kernel):
        assert bench.measured_traffic(rec["workload"], kernel) == rec["bytes_per_launch"]
    else:
        assert bench.measured_traffic(rec["workload"], kernel) is None


@pytest.mark.parametrize("extra", [("--graph",), ("--inplace",), ("--heads", "4"), ("--dtype", "f32")])
def test_cycle_mode_refuses_other_rope_options(monkeypatch, extra):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--cycle", *extra])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert "--cycle" in str(e.value.code)


def test_only_the_cpu_leg_runs_the_oracle():
    """bench.py imports the oracle (test infrastructure) only inside its CPU leg: the cpu_leg_*
    functions and the baseline timers they call."""
    import ast

    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    allowed = {"cpu_baseline", "neox_cpu_baseline"}
    for fn in [n for n in tree.body if isinstance(n, ast.FunctionDef)]:
        for node in ast.walk(fn):
            names = []
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            if any(n == "oracle" or n.startswith("oracle.") for n in names):
                assert fn.name.startswith("cpu_leg_") or fn.name in allowed, fn.name
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any("oracle" in ast.dump(n) for n in top)


def test_cpu_leg_compares_every_element():
    """The bench line's parity pass: the oracle over blocks of rows of every frame, compared with a
    result bit for bit -- the oracle's own output passes, and each planted difference is counted."""
    import numpy as np

    import oracle
    import workloads

    shape, split = (2, 3, 5, 7, 4, 32), (8, 8, 16)
    for dtype in (oracle.BF16, oracle.F32):
        q, _ = workloads.generate_custom(shape, dtype, seed=77)
        want = oracle.rope3d(q, dtype, split)
        assert bench.cpu_leg_compare_all(q, want, dtype, split, 10000.0, 3) == (0, None)
        bad = want.copy()
        raw = bad.view(np.uint32) if dtype == oracle.F32 else bad
        raw[1, 2, 4, 6, 3, 31] ^= 1
        raw[0, 0, 0, 0, 0, 0] ^= 2
        n, first = bench.cpu_leg_compare_all(q, bad, dtype, split, 10000.0, 3)
        assert n == 2 and first["index"] == [0, 0, 0, 0, 0, 0]


def test_neox_cpu_leg_compares_every_element():
    """The rotate-half bench line's parity pass over blocks of tokens: the oracle's own output
    passes with every element counted, and a planted difference is found and located."""
    import argparse

    import numpy as np
    import torch

    import oracle
    import oracle.neox as nx
    import workloads

    args = argparse.Namespace(cpu_threads=3, no_cpu_baseline=True, cpu_seconds=0.0)
    for key in ("n1", "n3"):
        w = workloads.NEOX_WORKLOADS[key]
        q, k, pos, cache = workloads.generate_neox(w)
        wq = nx.neox_rope(q, w.dtype, pos, cache, w.cache_dtype)
        wk = nx.neox_rope(k, w.dtype, pos, cache, w.cache_dtype)

        def as_torch(a):
            t = torch.from_numpy(a.view(np.int16) if w.dtype == oracle.BF16 else a.copy())
            return t.view(torch.bfloat16) if w.dtype == oracle.BF16 else t

        parity, cpu = bench.cpu_leg_neox(w, q, k, pos, cache, as_torch(wq), as_torch(wk), args)
        assert cpu is None
        assert parity["compared_elements"] == q.size + k.size and parity["mismatching_elements"] == 0
        bad = wk.copy()
        (bad.view(np.uint32) if w.dtype == oracle.F32 else bad)[w.tokens - 1, 1, 5] ^= 1
        parity, _ = bench.cpu_leg_neox(w, q, k, pos, cache, as_torch(wq), as_torch(bad), args)
        assert parity["mismatching_elements"] == 1
        assert parity["first_mismatch"]["tensor"] == "k" and parity["first_mismatch"]["index"] == [w.tokens - 1, 1, 5]
