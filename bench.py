"""Benchmark of the fused Q+K 3D RoPE on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 5] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic,
already-resident input: the cached table lookup (a hit after the first call),
the precheck, and the fused rotation of Q and K into fresh outputs
(torch.empty_like, as the decoder's wrapper does), i.e. one decoder block's
RoPE.  The default workload is the largest bf16 one: B=2, (T, H, W) =
(17, 68, 120), 32 heads, head_dim 96, split (32, 32, 32), N(0,1) values from
seed 4 (6.82 GB moved per step).

Printed: one JSON line.  value = algorithmic bytes per step / wall time per step
(GB/s).  roofline.achieved = algorithmic bytes per launch / the kernel's average
duration: the time between two HIP events recorded on the kernel's stream before
the first and after the last of the K timed launches, divided by K (the launches
run back to back; no marker sits between two kernels).  The CPU leg (the
cpu_leg_* functions, the only code here that runs the oracle, which is test
infrastructure) computes the oracle's result for the whole workload on a pool of
threads and compares every element of the GPU's timed outputs with it (parity;
in place: sampled tokens), and times the oracle on one core over a bounded
sample of the same workload, scaled to the same unit: cpu_baseline (skipped with
--no-cpu-baseline; the pool pass is reported under all_cores).

--op neox | patchify | unpatchify time the secondary kernels the same way
(200 warm-up and 200 timed launches of about 0.13 ms each by default), with
their own counter records and CPU-oracle baselines.
--op dit_freqs times the DiT frequency-grid kernel (launch-bound: roofline null).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused Q+K 3D RoPE achieved HBM GB/s (% of peak) + Gelem/s, bit-exact vs oracle"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
CSRC = os.path.join(ROOT, "rope_ltx3drope_amd", "csrc")
# each timed kernel: its source file and the local headers it includes
KERNEL_SOURCES = {
    "rope_fast": ("kernels.hip", "pair_math.h", "stream_store.h", "internal.h", "fastdiv.h"),
    "neox_fast": ("neox.hip", "stream_store.h", "internal.h"),
    "patch_lds": ("patchify.hip", "stream_store.h", "internal.h", "fastdiv.h"),
    "unpatch_lds": ("patchify.hip", "stream_store.h", "internal.h", "fastdiv.h"),
}


def traffic_file(kernel: str) -> str:
    """The committed rocprofv3 counter record of one kernel."""
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")


TRAFFIC_FILE = traffic_file("rope_fast")


def kernel_source_hash(kernel: str = "rope_fast") -> str:
    """Hash of a kernel's source files with comments and blank lines removed, so that a change of
    comments alone does not invalidate the committed counter measurements."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
        h.update(("\n".join(line for line in lines if line) + "\n").encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, kernel: str = "rope_fast"):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on this
    workload and on the kernel source that is built now (otherwise None)."""
    if kernel not in KERNEL_SOURCES:
        return None
    try:
        with open(traffic_file(kernel)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(kernel) or rec.get("workload") != workload_name:
        return None
    return rec.get("bytes_per_launch")


def pin_one_core():
    """Run the calling process on one core, so the CPU baseline states the threads it used."""
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50 for rope3d, 200 for the ~0.13 ms secondary kernels)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 20 for rope3d, 200 for the secondary kernels: "
                         "about 20 ms of GPU work either way, past the clock ramp seen after idle)")
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--grid", type=int, default=0, help="grid index inside the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="rope3d: threads of the oracle's pass over the whole workload that checks every output "
                         "element (default: the usable cores, at most 16)")
    ap.add_argument("--op", choices=("rope3d", "neox", "patchify", "unpatchify", "dit_freqs"), default="rope3d",
                    help="rope3d: the fused 3D RoPE (default); neox: the rotate-half RoPE with a gathered cache; "
                         "patchify / unpatchify: the stage-5 space-to-depth and its inverse")
    ap.add_argument("--patch-workload", default="p6")
    ap.add_argument("--neox-workload", default="n4")
    ap.add_argument("--dtype", choices=("auto", "f32", "bf16"), default="auto",
                    help="rope3d: run the workload's geometry in this dtype (auto: the workload's own)")
    ap.add_argument("--split", default="",
                    help="rope3d: dim_t,dim_h,dim_w instead of the workload's split (same head_dim)")
    ap.add_argument("--heads", type=int, default=0,
                    help="rope3d: this many heads instead of the workload's (e.g. one GPU's share under "
                         "head parallelism)")
    ap.add_argument("--graph", action="store_true",
                    help="rope3d: capture the K timed launches in one HIP graph and time its replay "
                         "(for the launch-bound small workloads); the default is eager launches")
    ap.add_argument("--reuse-outputs", action="store_true",
                    help="rope3d: write into output buffers allocated once per input set instead of fresh ones")
    ap.add_argument("--inplace", action="store_true",
                    help="rope3d: rotate Q and K in place instead of into fresh outputs")
    ap.add_argument("--cycle", action="store_true",
                    help="rope3d: one step = the workload's whole call sequence over its grids (workload 5: "
                         "(G1, G2, G3) x 4 from the table cache; workload 3: its 24 calls), fresh outputs")
    ap.add_argument("--rotate", type=int, default=0,
                    help="cycle through this many input/output sets (0: enough to exceed 2x the 256 MB "
                         "Infinity Cache, so every step streams from HBM)")
    args = ap.parse_args()
    short = args.op != "rope3d"
    if args.steps is None:
        args.steps = 200 if short else 50
    if args.warmup is None:
        args.warmup = 200 if short else 20
    if args.cpu_threads is None:
        try:
            args.cpu_threads = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            args.cpu_threads = min(16, os.cpu_count() or 1)
    if args.steps < 1 or args.warmup < 0 or args.rotate < 0:
        ap.error("--steps must be at least 1, --warmup and --rotate at least 0")
    return args


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the fused RoPE needs no communication; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    if args.op == "neox":
        return main_neox(args)
    if args.op in ("patchify", "unpatchify"):
        return main_patch(args)
    if args.op == "dit_freqs":
        return main_dit(args)
    if args.cycle:
        if args.graph or args.inplace or args.reuse_outputs or args.heads or args.split or args.dtype != "auto":
            raise SystemExit("--cycle times the workload as defined: no other rope3d option applies")
        return main_cycle(args)

    import numpy as np
    import torch

    import rope_ltx3drope_amd as rla
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    if args.dtype not in ("auto", w.dtype):
        # the same geometry, split, base, seed and value recipe in the other dtype
        w = dataclasses.replace(w, dtype=args.dtype, name=f"{w.name}_as_{args.dtype}")
    if args.split:
        split = tuple(int(x) for x in args.split.split(","))
        if len(split) != 3 or sum(split) != w.head_dim:
            raise SystemExit(f"--split needs three even widths summing to head_dim {w.head_dim}")
        w = dataclasses.replace(w, split=split, name=f"{w.name}_split{'_'.join(map(str, split))}")
    if args.heads:
        if args.heads < 1:
            raise SystemExit("--heads must be positive")
        w = dataclasses.replace(w, heads=args.heads, name=f"{w.name}_heads{args.heads}")
    gi = args.grid
    B, T, H, W, heads, D = w.shape(gi)
    numel = w.numel(gi)
    es = w.itemsize
    alg_bytes = w.algorithmic_bytes(gi)  # Q and K read once, written once
    elems = 2 * numel

    t0 = time.perf_counter()
    (q_np, k_np), = workloads.generate(w, [gi])
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s: {w.name} grid {gi} "
          f"shape {w.shape(gi)}", file=sys.stderr, flush=True)
    tdt = torch.bfloat16 if es == 2 else torch.float32
    if es == 2:
        q = torch.from_numpy(q_np.view(np.int16)).view(torch.bfloat16).to(dev)
        k = torch.from_numpy(k_np.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        q = torch.from_numpy(q_np).to(dev)
        k = torch.from_numpy(k_np).to(dev)
    assert q.dtype == tdt
    stream = torch.cuda.current_stream(dev)
    # input sets: one when Q+K already exceed the cache; otherwise enough copies that consecutive
    # steps never find their inputs in the 256 MB Infinity Cache
    mall = 256 << 20
    rotate = args.rotate or min(64, max(1, -(-4 * mall // alg_bytes)))
    sets = [(q, k)] + [(q.clone(), k.clone()) for _ in range(rotate - 1)]
    counter = [0]
    applied = [0] * rotate  # in-place mode: rotations applied to each input set so far
    # --reuse-outputs: one output pair per input set, allocated once (a serving loop's buffers)
    reused = [(torch.empty_like(q), torch.empty_like(k)) for _ in range(rotate)] if args.reuse_outputs else []

    def step():
        qi, ki = sets[counter[0] % rotate]
        applied[counter[0] % rotate] += 1
        counter[0] += 1
        tab = rla.tables_build(T, H, W, w.split, w.base, device=0)
        if args.inplace:
            rla.apply_qk(qi, ki, tab, inplace=True)
            tab.close()
            return qi, ki
        if args.reuse_outputs:
            qo, ko = reused[(counter[0] - 1) % rotate]
        else:
            qo = torch.empty_like(qi)
            ko = torch.empty_like(ki)
        rla.apply_qk(qi, ki, tab, qo, ko)
        tab.close()
        return qo, ko

    if args.inplace:
        if args.graph:
            raise SystemExit("--inplace and --graph are not combined")
        # an in-place call runs the fast kernel only for a configuration the gate already trusts:
        # one out-of-place call (into scratch outputs) runs the verification first
        with rla.tables_build(T, H, W, w.split, w.base, device=0) as tab:
            rla.apply_qk(q, k, tab, torch.empty_like(q), torch.empty_like(k))
        torch.cuda.synchronize()

    # the output blocks of rotate + 1 steps are reserved once, and the warmup keeps outputs alive
    # as the timed loop does (the last `rotate` sets): no device allocation inside the timed region
    if not (args.inplace or args.reuse_outputs or args.graph):
        reserve_outputs((q.shape, k.shape), q.dtype, dev, rotate + 1)
    settle_ms = settle_gpu(sets, stream)
    outs = []
    for _ in range(args.warmup):
        outs.append(step())
        if len(outs) > rotate:
            outs.pop(0)
    torch.cuda.synchronize()
    st = rla.stats()
    kernel = "rope_fast" if st["fast_launches"] > 0 and st["gate_disabled"] == 0 else "rope_plain"

    if args.graph:
        # the K steps' launches captured once into a HIP graph (tables and outputs fixed before
        # capture), then replayed: one untimed replay, one timed between two events
        outs.clear()
        outs_static = [(torch.empty_like(q), torch.empty_like(k)) for _ in range(rotate)]
        tab = rla.tables_build(T, H, W, w.split, w.base, device=0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                rla.apply_qk(*sets[i % rotate], tab, *outs_static[i % rotate])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        seg0 = device_segments(dev)
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        new_segments = device_segments(dev) - seg0
        wall = time.perf_counter() - t0
        tab.close()
        qo, ko = outs_static[(args.steps - 1) % rotate]
        last_in = (args.steps - 1) % rotate
        kernel_ms = [e0.elapsed_time(e1) / args.steps]
    else:
        # one pair of events around the K steps: the launches run back to back (the host needs
        # ~20 us per step, the kernel ~1 ms), and no marker sits between two kernels
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        seg0 = device_segments(dev)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            outs.append(step())
            if len(outs) > rotate:
                outs.pop(0)  # keep `rotate` output sets alive so the allocator cannot hand back a cached one
        e1.record(stream)
        torch.cuda.synchronize()
        new_segments = device_segments(dev) - seg0
        qo, ko = outs[-1]
        last_in = (args.steps + args.warmup - 1) % rotate
        wall = time.perf_counter() - t0
        kernel_ms = [e0.elapsed_time(e1) / args.steps]
    kavg_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = alg_bytes / (wall / args.steps) / 1e9
    achieved = alg_bytes / kavg_s / 1e9
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, kernel avg {kavg_s * 1e6:.1f} us, "
          f"{achieved:.0f} GB/s kernel", file=sys.stderr, flush=True)

    if not args.inplace:
        assert torch.equal(sets[last_in][0], q) and torch.equal(sets[last_in][1], k)
    copy_gbs = copy_ceiling(sets, stream)
    other_copies = platform_copies(sets[0], stream)
    parity, cpu = cpu_leg_rope3d(w, gi, q_np, k_np, qo, ko, applied[last_in] if args.inplace else 0, args)

    traffic = measured_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), inputs resident in HBM)",
        "config": {"workload": w.name, "B": B, "grid_THW": [T, H, W], "heads": heads, "head_dim": D,
                   "rope_dim_split": list(w.split), "base": w.base, "tokens": B * T * H * W,
                   "algorithmic_bytes_per_step": alg_bytes, "input_sets": rotate, "parallelism": "single GPU",
                   "launch": "hip_graph" if args.graph else "eager",
                   "outputs": "in_place" if args.inplace else ("reused" if args.reuse_outputs else "fresh")},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "gelem_per_s": round(elems / (wall / args.steps) / 1e9, 2),
        "kernel": kernel,
        "kernel_avg_us": round(kavg_s * 1e6, 2),
        "timed_region_device_allocations": new_segments,
        "gpu_settle_ms": round(settle_ms, 1),
        "copy_ceiling_GBps": None if copy_gbs is None else round(copy_gbs, 1),
        "pct_of_copy_ceiling": None if copy_gbs is None else round(100.0 * achieved / copy_gbs, 2),
        "platform_copies_GBps": other_copies,
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    emit(line)
    if parity["mismatching_elements"]:
        sys.exit(1)


def main_cycle(args):
    """The fused 3D RoPE over a workload's whole call sequence: one step = every call of the
    sequence, each on its own grid's inputs with fresh outputs, its tables from the cache (one
    build per grid, in the warmup)."""
    import numpy as np
    import torch

    import rope_ltx3drope_amd as rla
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    grids = sorted(set(w.calls))
    t0 = time.perf_counter()
    host = workloads.generate(w, grids)
    print(f"[bench] inputs of {len(grids)} grid(s) generated in {time.perf_counter() - t0:.1f} s: {w.name}",
          file=sys.stderr, flush=True)
    tdt = torch.bfloat16 if w.itemsize == 2 else torch.float32

    def to_dev(x):
        return (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if w.itemsize == 2
                else torch.from_numpy(x)).to(dev)

    inputs = {gi: (to_dev(q), to_dev(k)) for gi, (q, k) in zip(grids, host)}
    alg_pass = sum(w.algorithmic_bytes(gi) for gi in w.calls)
    elems_pass = sum(2 * w.numel(gi) for gi in w.calls)
    stream = torch.cuda.current_stream(dev)
    last = {}  # grid -> its latest outputs (the previous ones are released after the next call's allocation)

    def call(gi):
        q, k = inputs[gi]
        T, H, W = w.grids[gi]
        tab = rla.tables_build(T, H, W, w.split, w.base, device=0)
        qo, ko = torch.empty_like(q), torch.empty_like(k)
        rla.apply_qk(q, k, tab, qo, ko)
        tab.close()
        last[gi] = (qo, ko)

    def step():
        for gi in w.calls:
            call(gi)

    # two output sets per grid reserved up front: no device allocation inside the timed region
    for gi in grids:
        reserve_outputs((inputs[gi][0].shape, inputs[gi][1].shape), tdt, dev, 2)
    settle_ms = settle_gpu([inputs[grids[0]]], stream)
    rla.cache_clear()
    rla.stats_reset()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm = rla.stats()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    seg0 = device_segments(dev)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    new_segments = device_segments(dev) - seg0
    st = rla.stats()
    kernel = "rope_fast" if st["fast_launches"] > 0 and st["gate_disabled"] == 0 else "rope_plain"
    calls = args.steps * len(w.calls)
    gpu_s = e0.elapsed_time(e1) / 1e3
    achieved = alg_pass * args.steps / gpu_s / 1e9
    value = alg_pass / (wall / args.steps) / 1e9

    parity = {"compared_elements": 0, "mismatching_elements": 0, "tolerance_ulp": 0}
    for gi, (q_np, k_np) in zip(grids, host):  # every element of every grid's last outputs
        pg, _ = cpu_leg_rope3d(w, gi, q_np, k_np, *last[gi], 0, args, time_it=False)
        parity["compared_elements"] += pg["compared_elements"]
        parity["mismatching_elements"] += pg["mismatching_elements"]
    copy_gbs = copy_ceiling([inputs[grids[0]]], stream)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), inputs resident in HBM)",
        "config": {"workload": w.name + "_call_sequence", "B": w.B, "grids_THW": [list(g) for g in w.grids],
                   "call_sequence": list(w.calls), "heads": w.heads, "head_dim": w.head_dim,
                   "rope_dim_split": list(w.split), "base": w.base,
                   "algorithmic_bytes_per_step": alg_pass, "parallelism": "single GPU", "launch": "eager",
                   "outputs": "fresh"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "gelem_per_s": round(elems_pass / (wall / args.steps) / 1e9, 2),
        "kernel": kernel,
        "kernel_avg_us": round(gpu_s / calls * 1e6, 2),
        "timed_region_device_allocations": new_segments,
        "gpu_settle_ms": round(settle_ms, 1),
        "table_cache": {"warmup_misses": warm["cache_misses"], "warmup_hits": warm["cache_hits"],
                        "timed_misses": st["cache_misses"] - warm["cache_misses"],
                        "timed_hits": st["cache_hits"] - warm["cache_hits"]},
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "pct_of_copy_ceiling": round(100.0 * achieved / copy_gbs, 2),
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    emit(line)
    if parity["mismatching_elements"]:
        sys.exit(1)


def main_neox(args):
    """The rotate-half RoPE with a gathered cos/sin cache: one step = fresh outputs + one launch."""
    import numpy as np
    import torch

    import rope_ltx3drope_amd as rla
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.NEOX_WORKLOADS[args.neox_workload]
    q_np, k_np, pos_np, cache_np = workloads.generate_neox(w)

    def dev_t(x, dt):
        if dt == workloads.BF16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    q, k = dev_t(q_np, w.dtype), dev_t(k_np, w.dtype)
    pos, cache = torch.from_numpy(pos_np).to(dev), dev_t(cache_np, w.cache_dtype)
    alg = w.algorithmic_bytes()
    mall = 256 << 20
    rotate = args.rotate or min(64, max(1, -(-4 * mall // alg)))
    sets = [(q, k)] + [(q.clone(), k.clone()) for _ in range(rotate - 1)]
    stream = torch.cuda.current_stream(dev)
    reused = [(torch.empty_like(a), torch.empty_like(b)) for a, b in sets] if args.reuse_outputs else []
    if not args.reuse_outputs:
        reserve_outputs((q.shape, k.shape), q.dtype, dev, rotate + 1)
    settle_ms = settle_gpu(sets, stream)
    outs = []

    def step(i):
        qi, ki = sets[i % rotate]
        if args.reuse_outputs:
            qo, ko = reused[i % rotate]
        else:
            qo, ko = torch.empty_like(qi), torch.empty_like(ki)
        rla.neox_apply_qk(qi, ki, pos, cache, qo, ko)
        outs.append((qo, ko))
        if len(outs) > rotate:
            outs.pop(0)

    for i in range(args.warmup):  # outputs kept as in the timed loop: no allocation inside it
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    seg0 = device_segments(dev)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    new_segments = device_segments(dev) - seg0
    wall = time.perf_counter() - t0
    kavg = e0.elapsed_time(e1) / args.steps / 1e3  # launches run back to back: no marker between them
    qo, ko = outs[-1]
    st = rla.stats()
    kernel = "neox_fast" if st["fast_launches"] else "neox_plain"
    del outs
    copy_gbs = copy_ceiling(sets, stream)
    parity, cpu = cpu_leg_neox(w, q_np, k_np, pos_np, cache_np, qo, ko, args)
    line = {
        "metric": "rotate-half RoPE with gathered cos/sin cache, achieved HBM GB/s, bit-exact vs oracle",
        "value": round(alg / (wall / args.steps) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": w.key, "tokens": w.tokens, "q_heads": w.q_heads, "k_heads": w.k_heads,
                   "head_dim": w.head_dim, "max_position": w.max_position, "cache_dtype": w.cache_dtype,
                   "positions": w.positions, "algorithmic_bytes_per_step": alg, "input_sets": rotate,
                   "outputs": "reused" if args.reuse_outputs else "fresh"},
        "kernel": kernel,
        "kernel_avg_us": round(kavg * 1e6, 2),
        "timed_region_device_allocations": new_segments,
        "gpu_settle_ms": round(settle_ms, 1),
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "pct_of_copy_ceiling": round(100.0 * alg / kavg / 1e9 / copy_gbs, 2),
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(alg / kavg / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / kavg / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.key, kernel)},
        "cpu_baseline": cpu,
    }
    emit(line)
    if parity["mismatching_elements"]:
        sys.exit(1)


def main_dit(args):
    """LTX DiT RoPE frequency grid (theta 10000, dim 4096, 6 rope elements: 682 values) generated on
    the device by one kernel launch per call, float64 and float32 recipes: kernel time per call from
    two events around the K back-to-back launches, bit-exact against the oracle."""
    import numpy as np
    import torch

    import rope_ltx3drope_amd as rla

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    theta, dim, ne = 10000.0, 4096, 6
    per_call, wall_call, graph_us, mism = {}, {}, {}, 0
    for double in (True, False):
        for _ in range(args.warmup):
            rla.dit_freq_grid(theta, dim, ne, double, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            out = rla.dit_freq_grid(theta, dim, ne, double, device=dev)
        e1.record(stream)
        torch.cuda.synchronize()
        key = "f64" if double else "f32"
        wall_call[key] = (time.perf_counter() - t0) / args.steps
        per_call[key] = e0.elapsed_time(e1) / 1e3 / args.steps
        mism += cpu_leg_dit(theta, dim, ne, double, out.cpu().numpy())
        graph_us[key], out = dit_graph_us(theta, dim, ne, double, args.steps)
        mism += cpu_leg_dit(theta, dim, ne, double, out.cpu().numpy())
    oracle_us = cpu_leg_dit_time(theta, dim, ne)
    us = per_call["f64"] * 1e6
    line = {
        "metric": "LTX DiT RoPE frequency grid generated on the device, time per call, bit-exact vs oracle",
        "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_call["f64"] * 1e3, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic (fixed parameters)",
        "config": {"workload": "dit_freqs_theta1e4_dim4096_ne6", "values": dim // ne,
                   "f32_recipe_call_us": round(per_call["f32"] * 1e6, 3),
                   "f32_recipe_wall_us": round(wall_call["f32"] * 1e6, 2)},
        "kernel": "dit_freqs", "kernel_avg_us": round(graph_us["f64"], 3),
        "kernel_avg_us_f32": round(graph_us["f32"], 3),
        "kernel_time_note": "value: eager calls through the binding (a fresh output each), the events' interval "
                            "per call, which the host's per-call work sets; kernel_avg_us: the same launches "
                            "replayed from one HIP graph into one output, per launch",
        "parity": {"compared_elements": 2 * (dim // ne), "mismatching_elements": mism, "tolerance_ulp": 0},
        "roofline": None,
        "roofline_note": "682 values in 3 workgroups of one launch: bound by launch latency, not by HBM or "
                         "arithmetic throughput",
        "cpu_baseline": {"value": round(oracle_us, 2), "unit": "us", "cores": 1, "kind": "oracle",
                         "sample": "the float64 recipe, one whole grid per call (exact rationals and 60-digit "
                                   "decimals)"},
    }
    emit(line)
    if mism:
        sys.exit(1)


def dit_graph_us(theta, dim, ne, double, steps):
    """(microseconds per launch, output): `steps` launches of the DiT grid kernel into one
    preallocated output, captured in one HIP graph through the C ABI and replayed; the events
    around the replay hold no host work, so this is the kernel's own time plus the graph's gap
    between launches."""
    import ctypes

    import torch

    from rope_ltx3drope_amd import _lib

    L = _lib.lib()
    out = torch.empty(dim // ne, dtype=torch.float32, device="cuda:0")
    n = ctypes.c_int64(0)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sp = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            st = L.ltx3drope_dit_freq_grid(float(theta), dim, ne, int(double), out.data_ptr(), sp, ctypes.byref(n))
            if st != _lib.OK:
                raise RuntimeError(f"dit_freq_grid under capture: status {st}")
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps, out


def patch_kernel_name(fast: bool, inverse: bool) -> str:
    """The kernel the library picks for a call (it names none itself)."""
    if not fast:
        return "patch_plain"
    return "unpatch_lds" if inverse else "patch_lds"


def main_patch(args):
    """Space-to-depth (or its inverse) of a 5-D tensor: one step = a fresh output + one launch."""
    import numpy as np
    import torch

    import rope_ltx3drope_amd as rla
    import workloads

    dev = torch.device("cuda:0")
    shape, p, eb = workloads.PATCH_WORKLOADS[args.patch_workload]
    x_np = workloads.generate_patch(shape, eb, seed=6)
    signed = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[eb]
    x = torch.from_numpy(x_np.view(signed)).to(dev)
    inverse = args.op == "unpatchify"
    src = rla.patchify(x, p) if inverse else x
    fn = (lambda t: rla.unpatchify(t, p)) if inverse else (lambda t: rla.patchify(t, p))
    alg = 2 * x.numel() * eb
    mall = 256 << 20
    rotate = args.rotate or min(64, max(1, -(-4 * mall // alg)))
    sets = [src] + [src.clone() for _ in range(rotate - 1)]
    if args.reuse_outputs:  # one output per input set, allocated once
        out_like = x if inverse else rla.patchify(x, p)
        reused = [torch.empty_like(out_like) for _ in range(rotate)]
        del out_like
        fn_out = (lambda t, o: rla.unpatchify(t, p, out=o)) if inverse else (lambda t, o: rla.patchify(t, p, out=o))
    stream = torch.cuda.current_stream(dev)
    if not args.reuse_outputs:
        B_, C_, F_, H_, W_ = x.shape
        out_shape = x.shape if inverse else (B_, C_ * p * p, F_, H_ // p, W_ // p)
        reserve_outputs((out_shape,), x.dtype, dev, rotate + 1)
    settle_ms = settle_gpu([(t,) for t in sets], stream)
    outs = []

    def step(i):
        if args.reuse_outputs:
            outs.append(fn_out(sets[i % rotate], reused[i % rotate]))
        else:
            outs.append(fn(sets[i % rotate]))
        if len(outs) > rotate:
            outs.pop(0)

    for i in range(args.warmup):  # outputs kept as in the timed loop: no allocation inside it
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    seg0 = device_segments(dev)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    new_segments = device_segments(dev) - seg0
    wall = time.perf_counter() - t0
    kavg = e0.elapsed_time(e1) / args.steps / 1e3  # launches run back to back: no marker between them
    got = outs[-1].cpu().numpy().view(x_np.dtype)
    del outs
    copy_gbs = copy_ceiling([(t,) for t in sets], stream)
    del sets
    parity, cpu = cpu_leg_patch(x_np, p, inverse, got, alg, args)
    st = rla.stats()
    kernel = patch_kernel_name(st["fast_launches"] > 0, inverse)
    name = patch_workload_name(args.op, shape, p, eb)
    line = {
        "metric": f"{args.op} (stage-5 space-to-depth) achieved HBM GB/s, bit-exact vs oracle",
        "value": round(alg / (wall / args.steps) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": {1: "u8", 2: "bf16-bits", 4: "f32-bits", 8: "u64"}[eb],
        "data": "synthetic (seeded random bit patterns)",
        "config": {"workload": name, "key": args.patch_workload, "shape": list(shape), "p": p, "elem_bytes": eb,
                   "algorithmic_bytes_per_step": alg, "input_sets": rotate,
                   "outputs": "reused" if args.reuse_outputs else "fresh"},
        "kernel": kernel,
        "kernel_avg_us": round(kavg * 1e6, 2),
        "timed_region_device_allocations": new_segments,
        "gpu_settle_ms": round(settle_ms, 1),
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "pct_of_copy_ceiling": round(100.0 * alg / kavg / 1e9 / copy_gbs, 2),
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(alg / kavg / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / kavg / 1e9 / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, kernel)},
        "cpu_baseline": cpu,
    }
    emit(line)
    if parity["mismatching_elements"]:
        sys.exit(1)


def device_info() -> dict:
    """The GPU the line was measured on, as the HIP runtime reports it (through torch)."""
    import torch

    p = torch.cuda.get_device_properties(0)
    out = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "hbm_bytes": int(p.total_memory)}
    for key in ("L2_cache_size", "clock_rate", "memory_clock_rate", "memory_bus_width"):
        v = getattr(p, key, None)
        if v is not None:
            out[key] = int(v)
    return out


def emit(line: dict) -> None:
    """Prints the one JSON line, with the device it was measured on."""
    line["device"] = device_info()
    print(json.dumps(line), flush=True)


def device_segments(dev) -> int:
    """Device memory segments torch's caching allocator has obtained so far (each one a hipMalloc)."""
    import torch

    return int(torch.cuda.memory_stats(dev).get("segment.all.allocated", 0))


def settle_gpu(sets, stream, seconds: float = 0.1) -> float:
    """Runs the library's copy kernel over the input sets (into scratch tensors) for about `seconds`
    of GPU time before the warm-up steps, so that the timed region does not start while the clocks
    are still rising after the idle time of input generation (measured on MI355X: without it the
    first 10-20 ms of launches run 3-13 % slower).  No step of the op runs here.  Returns the
    milliseconds spent."""
    import torch

    import rope_ltx3drope_amd as rla

    tensors = [t for t in sets[0]]
    dsts = [torch.empty_like(t) for t in tensors]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spent = 0.0
    rounds = 1
    while spent < seconds * 1e3:
        e0.record(stream)
        for _ in range(rounds):
            for d, t in zip(dsts, tensors):
                rla.copy_bytes(d, t, t.numel() * t.element_size() // 16 * 16)
        e1.record(stream)
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        rounds = min(rounds * 2, 64)
    del dsts
    return spent


def reserve_outputs(shapes, dtype, dev, count: int) -> None:
    """Makes torch's caching allocator hold `count` sets of output blocks of these shapes: the
    timed loop keeps `rotate` sets alive and allocates one more per step, so with rotate + 1 sets
    cached no step inside the timed region needs a new device allocation."""
    import torch

    held = [[torch.empty(sh, dtype=dtype, device=dev) for sh in shapes] for _ in range(count)]
    del held


def copy_ceiling(sets, stream, reps_per_set: int = 10) -> float:
    """GB/s of the library's plain copy kernel on the same input sets: one step copies each
    tensor of one set into a scratch tensor of its size (one read stream and one write stream per
    launch, the fast kernels' launch shape and cache hints), timed like the kernel; bytes = each
    tensor read once and written once."""
    import torch

    import rope_ltx3drope_amd as rla

    bytes_per_step = sum(2 * t.numel() * t.element_size() for t in sets[0])

    dsts = [tuple(torch.empty_like(t) for t in sets[0]) for _ in range(min(len(sets), 2))]
    for i in range(3):
        for d, t in zip(dsts[i % len(dsts)], sets[i % len(sets)]):
            rla.copy_bytes(d, t)
    reps = reps_per_set * len(sets)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(reps):
        for d, t in zip(dsts[i % len(dsts)], sets[i % len(sets)]):
            rla.copy_bytes(d, t)
    c1.record(stream)
    torch.cuda.synchronize()
    return bytes_per_step / (c0.elapsed_time(c1) / reps / 1e3) / 1e9


def platform_copies(tensors, stream, reps: int = 10) -> dict:
    """GB/s of the platform's own device-to-device copies over the same tensors, beside the
    library's copy kernel: hipMemcpyAsync (torch's copy_ of a contiguous tensor of the same dtype,
    which HIP serves with its blit kernel) and torch's vectorized elementwise kernel (neg, one
    read and one write per element).  Shows whether the copy kernel's rate is the chip's streaming
    rate or an artefact of its own launch shape."""
    import torch

    dsts = [torch.empty_like(t) for t in tensors]
    nbytes = sum(2 * t.numel() * t.element_size() for t in tensors)
    out = {}
    for name, fn in (("hipMemcpyAsync_d2d", lambda d, t: d.copy_(t)),
                     ("torch_elementwise_neg", lambda d, t: torch.neg(t, out=d))):
        for _ in range(3):
            for d, t in zip(dsts, tensors):
                fn(d, t)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(reps):
            for d, t in zip(dsts, tensors):
                fn(d, t)
        c1.record(stream)
        torch.cuda.synchronize()
        out[name] = round(nbytes / (c0.elapsed_time(c1) / reps / 1e3) / 1e9, 1)
    del dsts
    return out


def patch_workload_name(op: str, shape, p: int, elem_bytes: int) -> str:
    dt = {1: "u8", 2: "bf16", 4: "f32", 8: "u64"}[elem_bytes]
    return f"{op}_{dt}_{'x'.join(str(d) for d in shape)}_p{p}"


# ---------------------------------------------------------------------------
# The CPU leg: the only code in this file that runs the oracle (test infrastructure).  It
# computes the oracle's result on a bounded sample of the workload, compares the GPU's timed
# outputs with it element by element (the line's "parity"), and, unless --no-cpu-baseline, times
# the oracle on the host cores over a longer sample (the line's "cpu_baseline").
# ---------------------------------------------------------------------------

def cpu_leg_rope3d(w, gi, q_np, k_np, qo, ko, rotations, args, time_it=True):
    """3D RoPE.  Parity: every element of the GPU outputs qo, ko against the oracle, computed over
    blocks of rows of each (batch, frame) by a pool of threads (that pass, timed, is also the
    all-cores CPU figure); in place (rotations > 0) the oracle applied that many times to 256
    sampled tokens instead.  Then, unless --no-cpu-baseline, the oracle timed on one core over whole
    (batch, frame) slabs.  Returns (parity, cpu_baseline or None)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    B, T, H, W, heads, D = w.shape(gi)
    if rotations:
        ids = workloads.sample_tokens(B * T * H * W, 256, seed=1234)
        idx = torch.from_numpy(ids).to(qo.device)
        tabs = oracle.grid_tables(T, H, W, w.split, w.base)
        coords = oracle.token_coords(ids, T, H, W)
        mism = 0
        for x_np, out in ((q_np, qo), (k_np, ko)):
            want = x_np.reshape(B * T * H * W, heads, D)[ids]
            for _ in range(rotations):
                want = oracle.apply_rope_tokens(want, w.dtype, coords, tabs, w.split)
            got = _host_bits(out.view(B * T * H * W, heads, D)[idx], w.itemsize)
            mism += int((got.view(want.dtype) != want).sum())
        parity = {"sampled_tokens": int(len(ids)), "mismatching_elements": mism, "tolerance_ulp": 0}
        all_cores = None
    else:
        threads = max(1, args.cpu_threads)
        t0 = time.perf_counter()
        mism, first = 0, None
        for x_np, out in ((q_np, qo), (k_np, ko)):
            m, f = cpu_leg_compare_all(x_np, _host_bits(out, w.itemsize), w.dtype, w.split, w.base, threads)
            mism += m
            first = first or f
        dt = time.perf_counter() - t0
        parity = {"compared_elements": int(2 * q_np.size), "mismatching_elements": mism, "tolerance_ulp": 0}
        if first:
            parity["first_mismatch"] = first
        n = 2 * q_np.size
        all_cores = {"value": round(n * 2 * w.itemsize / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
                     "gelem_per_s": round(n / dt / 1e9, 5), "seconds": round(dt, 2),
                     "sample": f"the whole workload once (Q and K, {n} elements), blocks of rows of each (batch, "
                               f"frame) on {threads} threads, compared with the GPU outputs (includes the "
                               "comparison)"}
    cpu = None
    if time_it and not args.no_cpu_baseline:
        cpu = cpu_baseline(w, gi, q_np, k_np, args.cpu_seconds)
        if all_cores is not None:
            cpu["all_cores"] = all_cores
    return parity, cpu


def _host_bits(t, itemsize: int):
    """A device tensor's contents on the host as raw uint16 (bf16) or float32 values."""
    import numpy as np
    import torch

    h = t.detach().cpu()
    return h.view(torch.int16).numpy().view(np.uint16) if itemsize == 2 else h.numpy()


def cpu_leg_compare_all(x_np, got_np, dtype, split, base, threads: int):
    """(mismatching elements, first mismatch or None): the oracle applied to every block of up to
    8 M elements (rows of one (batch, frame), a shard of the whole grid with the whole grid's
    tables) from a pool of threads, each block compared bit for bit with got_np."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    B, T, H, W, heads, D = x_np.shape
    tables = oracle.grid_tables(T, H, W, split, base)
    rows = max(1, min(H, (1 << 23) // (W * heads * D)))
    view = (lambda a: a.view(np.uint32)) if got_np.dtype == np.float32 else (lambda a: a)

    def block(job):
        b, t, h0 = job
        h1 = min(H, h0 + rows)
        want = oracle.rope3d(np.ascontiguousarray(x_np[b:b + 1, t:t + 1, h0:h1]), dtype, split, base,
                             tables=tables, offsets=(t, h0, 0), grid=(T, H, W))
        got = got_np[b:b + 1, t:t + 1, h0:h1]
        neq = view(got) != view(want)
        n = int(neq.sum())
        if not n:
            return 0, None
        i = tuple(int(v) for v in np.argwhere(neq)[0])
        return n, {"index": [b, t, h0 + i[2]] + list(i[3:]), "got": hex(int(view(got)[i])),
                   "want": hex(int(view(want)[i]))}

    jobs = [(b, t, h0) for b in range(B) for t in range(T) for h0 in range(0, H, rows)]
    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(block, jobs))
    return sum(n for n, _ in res), next((f for n, f in res if n), None)


def cpu_leg_neox(w, q_np, k_np, pos_np, cache_np, qo, ko, args):
    """Rotate-half RoPE.  Parity: every element of the GPU outputs qo, ko against the oracle,
    computed over blocks of consecutive tokens by a pool of threads; then, unless
    --no-cpu-baseline, the oracle timed on one core over consecutive chunks.  Returns (parity,
    cpu_baseline or None)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle.neox as nx

    threads = max(1, args.cpu_threads)
    mism, first = 0, None
    for name, x_np, out in (("q", q_np, qo), ("k", k_np, ko)):
        got_np = _host_bits(out, w.itemsize)
        view = (lambda a: a.view(np.uint32)) if got_np.dtype == np.float32 else (lambda a: a)
        step = max(1, (1 << 23) // (x_np.shape[1] * x_np.shape[2]))

        def block(t0, x_np=x_np, got_np=got_np, view=view, step=step, name=name):
            t1 = min(w.tokens, t0 + step)
            want = nx.neox_rope(np.ascontiguousarray(x_np[t0:t1]), w.dtype, pos_np[t0:t1], cache_np, w.cache_dtype)
            neq = view(got_np[t0:t1]) != view(want)
            n = int(neq.sum())
            if not n:
                return 0, None
            i = tuple(int(v) for v in np.argwhere(neq)[0])
            return n, {"tensor": name, "index": [t0 + i[0]] + list(i[1:]), "got": hex(int(view(got_np[t0:t1])[i])),
                       "want": hex(int(view(want)[i]))}

        with ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(block, range(0, w.tokens, step)))
        mism += sum(n for n, _ in res)
        first = first or next((f for n, f in res if n), None)
    parity = {"compared_elements": int(q_np.size + k_np.size), "mismatching_elements": mism, "tolerance_ulp": 0}
    if first:
        parity["first_mismatch"] = first
    cpu = None if args.no_cpu_baseline else neox_cpu_baseline(w, q_np, k_np, pos_np, cache_np, args.cpu_seconds)
    return parity, cpu


def cpu_leg_dit(theta, dim, ne, double, got) -> int:
    """DiT frequency grid: elements of the GPU's grid that differ from the oracle's, bit for bit."""
    import numpy as np

    import oracle.dit_freqs as df

    want = df.freq_grid(theta, dim, ne, double)
    return int((got.view(np.uint32) != want.view(np.uint32)).sum())


def cpu_leg_dit_time(theta, dim, ne) -> float:
    """The oracle's float64 recipe, repeated for about a second (at least once): microseconds per
    call."""
    import oracle.dit_freqs as df

    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 1.0:
        df.freq_grid(theta, dim, ne, True)
        reps += 1
    return (time.perf_counter() - t0) / reps * 1e6


def cpu_leg_patch(x_np, p, inverse, got, alg, args):
    """patchify / unpatchify: the oracle on the whole workload, compared element by element with
    the GPU's output; then, unless --no-cpu-baseline, the same call repeated on one core for about
    --cpu-seconds.  Returns (parity, cpu_baseline or None)."""
    import oracle.patchify as pf

    if inverse:
        want = x_np
        fn_cpu, src_cpu = pf.unpatchify, None if args.no_cpu_baseline else pf.patchify(x_np, p)
    else:
        fn_cpu, src_cpu = pf.patchify, x_np
    cpu, calls, cpu_s = None, 0, 0.0
    if not args.no_cpu_baseline:
        pin_one_core()
    while src_cpu is not None:
        t0 = time.perf_counter()
        res = fn_cpu(src_cpu, p)
        cpu_s += time.perf_counter() - t0
        calls += 1
        if not inverse and calls == 1:
            want = res
        del res
        if args.no_cpu_baseline or cpu_s >= args.cpu_seconds:
            break
    del src_cpu
    if not args.no_cpu_baseline:
        cpu = {"value": round(calls * alg / cpu_s / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "seconds": round(cpu_s, 2),
               "sample": f"the whole workload, {calls} {args.op} calls; numpy, one thread pinned to one core; "
                         f"CPU: {_cpu_model()}"}
    parity = {"compared_elements": int(got.size), "mismatching_elements": int((got != want).sum()),
              "tolerance_ulp": 0}
    return parity, cpu


def neox_cpu_baseline(w, q_np, k_np, pos_np, cache_np, target_s):
    """The rotate-half oracle, untuned, on consecutive 256-token chunks of the same inputs (Q and K),
    wrapping round to the first token, single thread, until about target_s seconds of CPU work are
    done; scaled to the kernel's algorithmic bytes per token."""
    import oracle.neox as nx

    pin_one_core()
    chunk, start, tokens = 256, 0, 0
    t0 = time.perf_counter()
    while True:
        sl = slice(start, min(start + chunk, w.tokens))
        for x in (q_np, k_np):
            nx.neox_rope(x[sl], w.dtype, pos_np[sl], cache_np, w.cache_dtype)
        tokens += sl.stop - sl.start
        start = sl.stop % w.tokens
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(w.algorithmic_bytes() * tokens / w.tokens / dt / 1e9, 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{tokens} tokens ({tokens / w.tokens:.2f} passes over the {w.tokens}-token workload) in "
                      f"{chunk}-token chunks, Q and K; numpy, one thread pinned to one core; CPU: {_cpu_model()}"}


def cpu_baseline(w, gi, q_np, k_np, target_s):
    """The oracle, untuned, on whole (batch, frame) slabs of the same inputs (Q and K), single thread
    pinned to one core, until about target_s seconds of CPU work are done (or every slab is)."""
    import numpy as np

    import oracle

    B, T, H, W, heads, D = w.shape(gi)
    pin_one_core()
    t0 = time.perf_counter()
    tabs = oracle.grid_tables(T, H, W, w.split, w.base)
    t_tab = time.perf_counter() - t0
    per_slab = 2 * H * W * heads * D
    done = 0
    slabs = 0
    t0 = time.perf_counter()
    while slabs < B * T:
        b, t = divmod(slabs, T)
        for x in (q_np, k_np):
            oracle.rope3d(np.ascontiguousarray(x[b:b + 1, t:t + 1]), w.dtype, w.split, w.base,
                          tables=_slice_tables(tabs, t))
        done += per_slab
        slabs += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0 + t_tab
    eps = done / dt
    return {"value": round(eps * 2 * w.itemsize / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "gelem_per_s": round(eps / 1e9, 5), "seconds": round(dt, 2),
            "sample": f"{slabs} of {B * T} (batch, frame) slabs, Q and K ({done} elements), plus the grid's "
                      f"table build; numpy, one thread pinned to one core; CPU: {_cpu_model()}"}


def _slice_tables(tabs, t):
    """Tables for a one-frame slab at frame t: the t table restricted to row t."""
    (ct, st), hpair, wpair = tabs
    return ((ct[t:t + 1], st[t:t + 1]), hpair, wpair)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
