#!/usr/bin/env python3
"""Benchmark of the MI355X NVFP4 grouped GEMM (one GPU).

One "step" is one grouped call (nvfp4_gg_run) over one set of synthetic inputs that
already sit in HBM.  The headline workload is the page's shape g=2, m=[128,384], n=4096,
k=1536; the other timed page shapes are reported under "shapes" in the same JSON line.

Timing protocol (per shape):
  * R input sets rotate so that R * bytes >= 1 GiB (no L2/MALL reuse across calls: "cold");
  * K calls are captured into one HIP graph (torch.cuda.CUDAGraph) and replayed after W
    warm-up calls; HIP events on the replay stream bracket the replay; avg per call = t/K;
  * a second figure re-runs the same K calls as plain launches (host launch overhead
    included), and a third uses one input set only ("warm");
  * "us_per_call_spread" gives min / median / max over the headline replay and 4 further
    replays of the same cold graph.
The roofline object prices the kernel against the fp16 MFMA dense peak (the path's
contraction runs on v_mfma_f32_32x32x16_f16) with the algorithmic flops per launch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--shapes c1,c2,c3,c4]
                       [--no-cpu-baseline] [--cold-only] [--calibrate-copy]
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
HEADLINE = "c1"
PAGE_US = {"c1": 10.5, "c2": 14.3, "c3": 45.0, "c4": 47.5}   # B200 timings printed on the page (context)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
COLD_BYTES = 1 << 30
SPREAD_REPLAYS = 4             # further timed replays of the cold graph, for min/median/max
KERNEL_SOURCE = os.path.join(ROOT, "precision_moe_nvfp4_amd", "csrc", "nvfp4_gg_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_nvfp4_gg_c1.md")
SHAPES_PROFILE = os.path.join(ROOT, "profiles", "kernel_traffic_mfma_nvfp4_gg_c2_c3_c4.md")


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


def recorded_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def recorded_shape_traffic():
    """HBM bytes per launch (read + write, counter-scaled) per page shape from the committed
    rocprofv3 summaries, if they were taken on the current kernel source; {} otherwise."""
    out = {}
    t = recorded_traffic()
    if t is not None:
        out[HEADLINE] = t
    if os.path.exists(SHAPES_PROFILE):
        text = open(SHAPES_PROFILE).read()
        h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
        if h and h.group(1) == kernel_source_hash():
            for m in re.finditer(r"^\| (c\d) \|[^|]*\|[^|]*\| ([0-9,]+) \| ([0-9,]+) \|", text, re.M):
                out[m.group(1)] = float(m.group(2).replace(",", "")) + float(m.group(3).replace(",", ""))
    return out


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


def time_shape(torch, gg, name, steps, warmup, dev, cold_only=False, blocked=False):
    cfg = shape_of(name)
    nbytes = algorithmic_bytes(cfg.m, cfg.n, cfg.k)
    flops = algorithmic_flops(cfg.m, cfg.n, cfg.k)
    R = max(1, math.ceil(COLD_BYTES / nbytes))
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

    cold_seq = [i % R for i in range(steps)]
    warm_seq = [0] * steps
    with torch.cuda.stream(stream):
        launches([i % R for i in range(warmup)])
    torch.cuda.synchronize()

    def graph_time(seq, extra=0):
        """Average per call of one timed replay of the captured sequence; with extra > 0 also
        the per-call averages of that many further replays (run-to-run spread)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            launches(seq)
        with torch.cuda.stream(stream):
            g.replay()   # warm replay
        torch.cuda.synchronize()
        times = []
        for _ in range(1 + extra):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1000.0 / len(seq))
        return times if extra else times[0]

    def direct_time(seq):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            launches(seq)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / len(seq)

    cold = graph_time(cold_seq, extra=SPREAD_REPLAYS)
    us_cold = cold[0]   # the headline: exactly one timed replay of the K calls
    spread = sorted(cold)
    us_direct = None if cold_only else direct_time(cold_seq)
    us_warm = None if cold_only else graph_time(warm_seq)
    t_roof_us = max(nbytes / (PEAK_HBM_GBS * 1e3), flops / (PEAK_F16_TFLOPS * 1e6))
    res = {
        "us_per_call": round(us_cold, 3),
        "us_per_call_direct_launch": None if us_direct is None else round(us_direct, 3),
        "us_per_call_warm": None if us_warm is None else round(us_warm, 3),
        "us_per_call_spread": {"min": round(spread[0], 3), "median": round(spread[len(spread) // 2], 3),
                               "max": round(spread[-1], 3), "replays": len(spread)},
        "eff_tflops": round(flops / us_cold / 1e6, 1),
        "eff_hbm_tbs": round(nbytes / us_cold / 1e6, 3),
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": flops,
        "roofline_us_f16": round(t_roof_us, 3),
        "pct_roofline": round(100.0 * t_roof_us / us_cold, 1),
        "bound": "mfma" if flops / (PEAK_F16_TFLOPS * 1e6) >= nbytes / (PEAK_HBM_GBS * 1e3) else "hbm",
        "rotating_sets": R,
        "grid": info.grid, "block": info.block, "tile": [info.tile_m, info.tile_n],
        "scale_layout": "blocked128x4" if blocked else "row-major",
        "page_b200_us": PAGE_US.get(name),
    }
    del sets, Cs, args
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name):
    """The oracle as it stands, timed on the host cores: whole headline calls, repeated for
    about 10 s of CPU work (at most 30 s), median per call."""
    import oracle
    from synthetic import CONFIGS, make_inputs
    cfg = CONFIGS[name]
    inp = make_inputs(cfg.m, cfg.n, cfg.k, cfg.seed)
    times = []
    t_start = time.perf_counter()
    while (time.perf_counter() - t_start) < 10.0 and len(times) < 1000:
        t0 = time.perf_counter()
        oracle.grouped_inputs(inp, want_abs=False)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > 30.0:
            break
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
                    help="time only the cold graph replays (for profiler runs whose kernel "
                         "average should match the reported value)")
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
        shapes[nm] = time_shape(torch, gg, nm, a.steps, a.warmup, dev, cold_only=a.cold_only)
        print(f"bench: {nm} -> {shapes[nm]}", file=sys.stderr, flush=True)
    if not a.cold_only:
        # the headline workload again with its scales in the 128x4 blocked layout
        nm = HEADLINE + "_blocked_scales"
        print(f"bench: timing {nm}", file=sys.stderr, flush=True)
        shapes[nm] = time_shape(torch, gg, HEADLINE, a.steps, a.warmup, dev, cold_only=True, blocked=True)
        shapes[nm]["page_b200_us"] = None
        print(f"bench: {nm} -> {shapes[nm]}", file=sys.stderr, flush=True)
    traffic = recorded_shape_traffic()
    for nm, res in shapes.items():
        tb = traffic.get(nm)
        res["counter_traffic_bytes"] = tb
        res["counter_hbm_tbs"] = None if tb is None else round(tb / res["us_per_call"] / 1e6, 3)
    head = shapes[HEADLINE]
    cfg = CONFIGS[HEADLINE]
    us = head["us_per_call"]
    achieved = head["algorithmic_flops"] / us / 1e6  # TFLOP/s
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
                   "timing": "cold: rotating input sets >= 1 GiB, K calls in one HIP graph, HIP events"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": recorded_traffic(),
                     "kernel": "nvfp4gg::nvfp4_gg_persistent", "kernel_source_sha256_16": kernel_source_hash()},
        "shapes": shapes,
    }
    if not a.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(HEADLINE)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
