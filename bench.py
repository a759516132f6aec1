#!/usr/bin/env python3
"""Benchmark of the MI355X NVFP4 grouped GEMM (one GPU).

One "step" is one grouped call (nvfp4_gg_run) over one set of synthetic inputs that
already sit in HBM.  The headline workload is the largest of the page's timed shapes,
g=8, m=[80,176,128,72,64,248,96,160], n=4096, k=7168; the other timed shapes are reported
under "shapes" in the same JSON line, each with its own roofline and CPU-oracle baseline.

Timing protocol (per shape):
  * R input sets rotate so that R * bytes >= 1 GiB (no L2/MALL reuse across calls: "cold");
    the captured sequence holds max(K, R) calls, so every replay rotates through all R
    sets whatever K is;
  * the calls are captured into one HIP graph (torch.cuda.CUDAGraph) and replayed after W
    warm-up calls and one untimed replay; HIP events on the replay stream bracket each of
    5 timed replays; per-call time = replay time / calls;
  * the headline is the median of the 5 replays (min and max reported beside it);
  * with --full, a direct-launch figure (host launch overhead included) and a one-set
    ("warm") figure are added.
The roofline object prices the kernel against the fp16 MFMA dense peak (the path's
contraction runs on v_mfma_f32_32x32x16_f16) with the algorithmic flops per launch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--shapes c1,c2,c3,c4]
                       [--no-cpu-baseline] [--cold-only] [--full] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per grouped call + achieved HBM TB/s & eff. TFLOP/s (% roofline) per shape"
HEADLINE = "c4"
PAGE_US = {"c1": 10.5, "c2": 14.3, "c3": 45.0, "c4": 47.5}   # B200 timings printed on the page (context)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
COLD_BYTES = 1 << 30
REPLAYS = 5                    # timed replays of the cold graph: median (headline), min, max
KERNEL_SOURCE = os.path.join(ROOT, "precision_moe_nvfp4_amd", "csrc", "nvfp4_gg_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_nvfp4_gg_units.md")


DENSE = "8192:4096:4096"


def algorithmic_bytes(m, n, k):
    """Each operand byte read once, C written once: A + B + SFA + SFB + C(fp16)."""
    sm, g = sum(m), len(m)
    return sm * (k // 2) + g * n * (k // 2) + sm * (k // 16) + g * n * (k // 16) + 2 * sm * n


def algorithmic_flops(m, n, k):
    return 2 * sum(m) * n * k


def kernel_source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_shape_traffic():
    """HBM bytes per launch (read + write, counter-scaled) per shape from the committed
    rocprofv3 summary, if it was taken on the current kernel source; {} otherwise."""
    out = {}
    if not os.path.exists(TRAFFIC_FILE):
        return out
    text = open(TRAFFIC_FILE).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not h or h.group(1) != kernel_source_hash():
        return out
    for m in re.finditer(r"^\| (\S+) \|[^|]*\| ([0-9,]+) \| ([0-9,]+) \|", text, re.M):
        out[m.group(1)] = float(m.group(2).replace(",", "")) + float(m.group(3).replace(",", ""))
    return out


def cold_sequence(steps, nbytes):
    """Input-set indices of one timed replay: R sets with R * nbytes >= 1 GiB, each call the
    next set, max(steps, R) calls so that every replay touches all R sets."""
    R = max(1, math.ceil(COLD_BYTES / nbytes))
    return [i % R for i in range(max(steps, R))], R


def shape_of(name):
    """A page workload by name, or a custom shape "m0/m1/...:n:k" (diagnostics only)."""
    from synthetic import CONFIGS, GroupedShape
    if name in CONFIGS:
        return CONFIGS[name]
    ms, n, k = name.split(":")
    return GroupedShape(name, tuple(int(x) for x in ms.split("/")), int(n), int(k))


def make_sets(torch, gg, name, R, dev):
    """Set 0 is the seeded numpy workload (identical to the parity tests); sets 1..R-1 are
    drawn on the device with the same distribution (uniform bytes, scale codes 0x08..0x20)."""
    from synthetic import SCALE_CODE_HI, SCALE_CODE_LO, make_inputs
    cfg = shape_of(name)
    inp = make_inputs(cfg.m, cfg.n, cfg.k, cfg.seed)
    sets = []
    A, B, SFA, SFB = gg.device_operands(inp.A, inp.B, inp.SFA, inp.SFB, dev)
    sets.append((A, B, SFA, SFB))
    for r in range(1, R):
        gen = torch.Generator(device=dev)
        gen.manual_seed(cfg.seed + r)
        rnd = lambda shape: torch.randint(0, 256, shape, dtype=torch.uint8, device=dev, generator=gen)
        sc = lambda shape: torch.randint(SCALE_CODE_LO, SCALE_CODE_HI + 1, shape, dtype=torch.uint8,
                                         device=dev, generator=gen)
        sets.append(([rnd((mi, cfg.k // 2)) for mi in cfg.m], [rnd((cfg.n, cfg.k // 2)) for _ in cfg.m],
                     [sc((mi, cfg.k // 16)) for mi in cfg.m], [sc((cfg.n, cfg.k // 16)) for _ in cfg.m]))
    Cs = [[torch.empty((mi, cfg.n), dtype=torch.float16, device=dev) for mi in cfg.m] for _ in range(R)]
    return cfg, sets, Cs


def to_blocked(torch, gg, scales, k, dev):
    """Row-major scale tensors -> 128x4 blocked copies, converted by the library."""
    out = []
    for s in scales:
        rows = s.shape[0]
        d = torch.empty((max(gg.nvfp4_gg_blocked_scale_bytes(rows, k), 1),), dtype=torch.uint8, device=dev)
        gg.nvfp4_gg_scales_to_blocked(d, s, rows, k)
        out.append(d)
    return out


def time_shape(torch, gg, name, steps, warmup, dev, full=False, blocked=False):
    cfg = shape_of(name)
    nbytes = algorithmic_bytes(cfg.m, cfg.n, cfg.k)
    flops = algorithmic_flops(cfg.m, cfg.n, cfg.k)
    cold_seq, R = cold_sequence(steps, nbytes)
    cfg, sets, Cs = make_sets(torch, gg, name, R, dev)
    if blocked:
        # the same scale values in the 128x4 blocked layout (converted before timing)
        sets = [(A, B, to_blocked(torch, gg, SFA, cfg.k, dev), to_blocked(torch, gg, SFB, cfg.k, dev))
                for (A, B, SFA, SFB) in sets]
        torch.cuda.synchronize()
    plan = gg.nvfp4_gg_plan(cfg.m, cfg.n, cfg.k, scale_layout=gg.SCALES_BLOCKED if blocked else gg.SCALES_ROW_MAJOR)
    info = gg.nvfp4_gg_plan_info(plan)
    args = [gg.RunArgs(len(cfg.m), *sets[r], Cs[r]) for r in range(R)]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def launches(seq):
        h = stream.cuda_stream
        for r in seq:
            gg.nvfp4_gg_run(plan, args=args[r], stream=h)

    with torch.cuda.stream(stream):
        launches([i % R for i in range(warmup)])
    torch.cuda.synchronize()

    def graph_times(seq, replays):
        """Per-call averages of `replays` timed replays of the captured sequence (after one
        untimed replay)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            launches(seq)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1000.0 / len(seq))
        return sorted(times)

    def direct_time(seq):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            launches(seq)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / len(seq)

    cold = graph_times(cold_seq, REPLAYS)
    us = cold[len(cold) // 2]   # the headline: median of the timed replays
    us_direct = direct_time(cold_seq) if full else None
    us_warm = graph_times([0] * max(steps, 1), 3)[1] if full else None
    t_roof_us = max(nbytes / (PEAK_HBM_GBS * 1e3), flops / (PEAK_F16_TFLOPS * 1e6))
    achieved = flops / us / 1e6
    res = {
        "us_per_call": round(us, 3),
        "us_per_call_spread": {"min": round(cold[0], 3), "median": round(us, 3), "max": round(cold[-1], 3),
                               "replays": len(cold)},
        "us_per_call_direct_launch": None if us_direct is None else round(us_direct, 3),
        "us_per_call_warm": None if us_warm is None else round(us_warm, 3),
        "eff_tflops": round(achieved, 1),
        "eff_hbm_tbs": round(nbytes / us / 1e6, 3),
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": flops,
        "roofline_us_f16": round(t_roof_us, 3),
        "pct_roofline": round(100.0 * t_roof_us / us, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4)},
        "calls_per_replay": len(cold_seq),
        "rotating_sets": R,
        "rotated_bytes": R * nbytes,
        "grid": info.grid, "block": info.block, "units": info.total_tiles,
        "unit_shapes": sorted({(info.unit_rows[s], info.unit_cols[s]) for s in range(len(cfg.m)) if info.unit_rows[s]}),
        "scale_layout": "blocked128x4" if blocked else "row-major",
        "page_b200_us": PAGE_US.get(name),
    }
    del sets, Cs, args
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, budget_s=8.0):
    """The oracle as it stands, timed on the host cores: whole calls of the workload,
    repeated for about `budget_s` seconds of CPU work (at least one call), median per call."""
    import oracle
    cfg = shape_of(name)
    from synthetic import make_inputs
    inp = make_inputs(cfg.m, cfg.n, cfg.k, cfg.seed)
    times = []
    t_start = time.perf_counter()
    while not times or ((time.perf_counter() - t_start) < budget_s and len(times) < 1000):
        t0 = time.perf_counter()
        oracle.grouped_inputs(inp, want_abs=False)
        times.append(time.perf_counter() - t0)
    times.sort()
    us = times[len(times) // 2] * 1e6
    return {"value": round(us, 1), "unit": "us", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{len(times)} full {name} grouped calls (g={cfg.g}, n={cfg.n}, k={cfg.k}) in "
                      f"{time.perf_counter() - t_start:.1f} s, median; packed inputs to fp16 C, decode included; "
                      f"host CPU: {host_cpu_model()}"}


def host_cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calibrate_copy(torch):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # c1..c4: the grouped workloads; DENSE: one large group (g = 1, m = 8192, n = k = 4096)
    ap.add_argument("--shapes", default="c1,c2,c3,c4," + DENSE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--cold-only", action="store_true",
                    help="time only the cold graph replays of the listed shapes (no blocked-scale "
                         "line), e.g. for profiler runs whose kernel average should match the value")
    ap.add_argument("--full", action="store_true", help="also time direct launches and one warm input set")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: --gpus {a.gpus} is not supported: this NVFP4 grouped GEMM runs on one GPU "
              "(no sharding or collectives); run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    import precision_moe_nvfp4_amd as gg
    from synthetic import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if a.calibrate_copy:
        calibrate_copy(torch)
        return
    names = [s for s in a.shapes.split(",") if s]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    shapes = {}
    for nm in names:
        print(f"bench: timing {nm} {shape_of(nm)}", file=sys.stderr, flush=True)
        shapes[nm] = time_shape(torch, gg, nm, a.steps, a.warmup, dev, full=a.full)
        print(f"bench: {nm} -> {shapes[nm]}", file=sys.stderr, flush=True)
    if not a.cold_only:
        # the headline workload again with its scales in the 128x4 blocked layout
        nm = HEADLINE + "_blocked_scales"
        print(f"bench: timing {nm}", file=sys.stderr, flush=True)
        shapes[nm] = time_shape(torch, gg, HEADLINE, a.steps, a.warmup, dev, blocked=True)
        shapes[nm]["page_b200_us"] = None
        print(f"bench: {nm} -> {shapes[nm]}", file=sys.stderr, flush=True)
    traffic = recorded_shape_traffic()
    for nm, res in shapes.items():
        tb = traffic.get(nm)
        res["roofline"]["traffic"] = tb
        res["counter_hbm_tbs"] = None if tb is None else round(tb / res["us_per_call"] / 1e6, 3)
    if not a.no_cpu_baseline:
        for nm in names:
            if nm in PAGE_US:
                print(f"bench: timing the CPU oracle on {nm}", file=sys.stderr, flush=True)
                shapes[nm]["cpu_baseline"] = cpu_baseline(nm)
    head = shapes[HEADLINE]
    cfg = CONFIGS[HEADLINE]
    us = head["us_per_call"]
    line = {
        "metric": METRIC,
        "value": us,
        "unit": "us",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(us / PAGE_US[HEADLINE], 3),
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"NVFP4 grouped GEMM g={cfg.g} m={list(cfg.m)} n={cfg.n} k={cfg.k} seed={cfg.seed}",
                   "g": cfg.g, "m": list(cfg.m), "n": cfg.n, "k": cfg.k,
                   "timing": f"cold: {head['rotating_sets']} rotating input sets ({head['rotated_bytes']} bytes) per "
                             f"replay of {head['calls_per_replay']} calls in one HIP graph, median of "
                             f"{head['us_per_call_spread']['replays']} replays, HIP events"},
        "roofline": dict(head["roofline"], kernel="nvfp4gg::nvfp4_gg_units",
                         kernel_source_sha256_16=kernel_source_hash()),
        "shapes": shapes,
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
