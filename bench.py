"""Benchmark of the fused LiteLinear forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dit_r64] [--gpus 1]

One step is one litelinear_forward (all kernels of the path) over one batch
of seeded synthetic inputs already resident in HBM.  Several copies of the
inputs and outputs are rotated so that the working set exceeds the 256 MB
Infinity Cache and every step reads its operands from HBM.

Prints ONE JSON line with:
  value / unit      whole-step throughput in TFLOP/s of algorithmic work
                    (2 M (in out + r in + r out) flops per step);
  roofline          the dominant kernel's achieved rate against the MI355X
                    peak for its bound (dense bf16 matrix cores, 2.5 PFLOP/s,
                    or HBM, 8 TB/s), from HIP events recorded on the launch
                    stream around every launch of that kernel;
  cpu_baseline      the float64 CPU oracle timed on a sample of rows of the
                    same workload, on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth
MALL_BYTES = 256 << 20      # Infinity Cache


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="dit_r64")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--copies", type=int, default=0, help="rotating input/output copies (0: auto)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--path", default="auto", choices=["auto", "skinny", "tiled"])
    p.add_argument("--split-k", type=int, default=0, help="skinny path: K-slice hint (0: automatic)")
    p.add_argument("--t-splits", type=int, default=0, help="tiled path: K slices per T block (0: automatic)")
    return p.parse_args()


def kernel_flops_bytes(w, kernel: str):
    """Algorithmic flops and bytes one launch of `kernel` is charged with.

    Both the tiled kernel and the skinny kernel compute the whole forward in
    one launch: 2 M (in out + r in + r out) flops, and every input read once
    plus y written once.  The A-padding copy (ranks not a multiple of 8) moves
    2 out r bytes in and 2 out r_pad bytes out."""
    if kernel == "pad_a":
        r_pad = -(-w.rank // 64) * 64
        return 0, 2 * w.out_features * (w.rank + r_pad)
    return w.flops, w.bytes


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} / WORLD_SIZE {world} is not supported "
              "(every MI355X box here has one GPU; the forward's rows shard with no communication, "
              "so N GPUs give N times this figure)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rank_fp8_residual_amd import Handle, Kernel, Option, Path
    from rank_fp8_residual_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    w = wl.WORKLOADS[args.workload]
    log("workload", w)
    t0 = time.time()
    d = wl.make_inputs(w, seed=args.seed)
    log(f"inputs drawn in {time.time() - t0:.1f}s")

    per_copy = w.bytes
    copies = args.copies or max(2, min(64, math.ceil(4 * MALL_BYTES / per_copy)))
    sets = []
    for c in range(copies):
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
        g["y"] = torch.empty((w.M, w.out_features), dtype=torch.bfloat16, device=dev)
        sets.append(g)
    torch.cuda.synchronize()
    log(f"{copies} rotating copies resident ({copies * per_copy / 2**20:.0f} MiB)")

    h = Handle(0)
    h.set_option(Option.PATH, {"auto": Path.AUTO, "skinny": Path.SKINNY, "tiled": Path.TILED}[args.path])
    h.set_option(Option.SPLIT_K, args.split_k)
    h.set_option(Option.T_SPLITS, args.t_splits)

    def step(i):
        g = sets[i % copies]
        h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=g["y"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    gbs = w.bytes / (ms_step * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {ms_step * 1e3:.2f} us/step, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s")

    # Per-kernel times: HIP events the library records on the launch stream.
    h.set_option(Option.PROFILE, 1)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kt = {}
    for name, kind in (("pad_a", Kernel.PAD_A), ("main", Kernel.MAIN), ("skinny", Kernel.SKINNY)):
        ms, n = h.kernel_time(kind, reset=True)
        if n:
            kt[name] = ms / n
    h.set_option(Option.PROFILE, 0)
    dom = max(kt, key=kt.get)
    fl, by = kernel_flops_bytes(w, dom)
    dur_s = kt[dom] * 1e-3
    ai = fl / by
    if ai > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(fl / dur_s / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / dur_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = {"main": "fused_kernel (tiled path)", "pad_a": "pad_rows_kernel",
                      "skinny": "skinny_kernel"}[dom]
    roof["kernel_us"] = {k: round(v * 1e3, 2) for k, v in kt.items()}
    log("per-kernel us", roof["kernel_us"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, d, sets[0], args.cpu_seconds)

    line = {
        "metric": "fused LiteLinear TFLOP/s and HBM GB/s vs roofline, M=3630 in=2048 out=8192 r=64"
        if args.workload == "dit_r64" else f"fused LiteLinear TFLOP/s and HBM GB/s vs roofline, {args.workload}",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: M={w.M} in={w.in_features} out={w.out_features} r={w.rank}; "
                        "x/A/B/bias bf16, Q e4m3fn with per-tensor scale, y bf16",
            "M": w.M, "in": w.in_features, "out": w.out_features, "r": w.rank,
            "rotating_copies": copies, "hbm_GBps": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "flops_per_step": w.flops, "bytes_per_step": w.bytes,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, d, g, target_s):
    """Time the float64 CPU oracle on a bounded sample of rows of the workload."""
    import numpy as np
    import torch

    import oracle

    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))
    row_flops = 2 * (w.in_features * w.out_features + w.rank * (w.in_features + w.out_features))
    probe = min(w.M, max(threads, 8))
    rows = np.linspace(0, w.M - 1, probe).astype(np.int64)
    t = time.time()
    oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows, threads=threads)
    dt = max(time.time() - t, 1e-6)
    n = int(min(w.M, max(probe, probe * target_s / dt)))
    rows = np.unique(np.linspace(0, w.M - 1, n).astype(np.int64))
    log(f"cpu baseline: oracle on {rows.size} rows with {threads} threads")
    t = time.time()
    y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows, threads=threads)
    dt = time.time() - t
    value = rows.size * row_flops / dt / 1e12
    # parity of the GPU output on the same rows (bf16-output gates)
    from tests import parity
    ys = parity.to_f64(g["y"][torch.from_numpy(rows).to(g["y"].device)])
    m = parity.metrics(ys, y_ref)
    ok = True
    try:
        parity.check(ys, y_ref, out_f32=False)
    except AssertionError:
        ok = False
    log(f"cpu baseline: {dt:.1f}s, {value * 1e3:.2f} GFLOP/s; parity on sample ok={ok}")
    try:
        cpu_model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        cpu_model = "unknown"
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows.size} of {w.M} rows (all {w.out_features} outputs each), float64, "
                      f"{dt:.1f} s on {cpu_model}",
            "seconds": round(dt, 2),
            "parity_on_sample": {"ok": ok, "max_over_rms": round(m["max_over_rms"], 5),
                                 "rel_l1": round(m["rel_l1"], 6)}}


if __name__ == "__main__":
    main()
