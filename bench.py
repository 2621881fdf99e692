"""Benchmark of the fused LiteLinear forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dit_r64] [--gpus 1]

One step is one litelinear_forward (every kernel of the path) over one batch
of seeded synthetic inputs already resident in HBM.  Several copies of the
inputs and outputs are rotated so that the working set exceeds the 256 MB
Infinity Cache and every step reads its operands from HBM.

Prints ONE JSON line with:
  value / unit      whole-step throughput in TFLOP/s of algorithmic work
                    (2 M (in out + r in + r out) flops per step);
  roofline          the dominant kernel's achieved rate against the MI355X
                    peak for its bound (dense bf16 matrix cores, 2.5 PFLOP/s,
                    or HBM, 8 TB/s): algorithmic work per launch over the
                    kernel's time per launch, from HIP events on the launch
                    stream around the timed region (or, when a step launches
                    more than one kernel, around every launch of that one);
                    `traffic` is the kernel's measured HBM bytes per launch
                    when a counter record for the current kernel sources is
                    committed under profiles/ (else null);
  cpu_baseline      the float64 CPU oracle timed on a sample of rows of the
                    same workload, on this host's cores;
  workloads         a shorter measurement of every other workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth
MALL_BYTES = 256 << 20      # Infinity Cache
COPY_PROBE_BYTES = 256 << 20
KERNEL_NAMES = {"main": "fused_kernel", "pad_a": "pad_rows_kernel", "skinny": "skinny_kernel",
                "quant": "quant_rows_kernel"}
# compute-bound workloads also measured with e4m3fn activations in the summary
ACT8_SUMMARY = ("llm", "dit_r32", "dit_r64", "dit_r512", "large")
# weights whose decomposition step (residual + e4m3fn quantisation) is timed
CONVERT_SUMMARY = ("dit_r64", "large")
PAIR_SUMMARY = ("llm", "dit_r64")  # shared-B pairs of these shapes
HEADLINE = "dit_r64"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--ramp-ms", type=float, default=400.0,
                   help="untimed steps for at least this long before the warm-up and the timed region "
                        "(the clocks ramp up under load)")
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--copies", type=int, default=0, help="rotating input/output copies (0: auto)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-summary", action="store_true", help="skip the other workloads")
    p.add_argument("--no-read-probe", action="store_true", help="skip the 64 MiB HBM read-ceiling probe")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 256 MiB device copy (reference kernel for HBM counters)")
    p.add_argument("--path", default="auto", choices=["auto", "skinny", "tiled"])
    p.add_argument("--split-k", type=int, default=0, help="skinny path: K-slice hint (0: automatic)")
    p.add_argument("--t-splits", type=int, default=0, help="tiled path: K slices per T block (0: automatic)")
    p.add_argument("--t-launch", type=int, default=0, choices=[0, 1, 2],
                   help="tiled path: how T is computed (the T_LAUNCH option; 0: automatic)")
    p.add_argument("--act-fp8", action="store_true",
                   help="e4m3fn activations for the residual product (LITELINEAR_OPT_ACT_FP8)")
    return p.parse_args()


def kernel_flops_bytes(w, kernel: str):
    """Algorithmic flops and bytes one launch of `kernel` is charged with.

    The tiled kernel and the skinny kernel each compute the whole forward in
    one launch: 2 M (in out + r in + r out) flops, and every input read once
    plus y written once.  The A-padding copy (ranks not a multiple of 8)
    moves 2 out r bytes in and 2 out r_pad bytes out."""
    if kernel == "pad_a":
        r_pad = -(-w.rank // 64) * 64
        return 0, 2 * w.out_features * (w.rank + r_pad)
    if kernel == "quant":  # x read, codes and row scales written
        return 0, 3 * w.M * w.in_features + 4 * w.M
    return w.flops, w.bytes


def mfma_peak(w, act8: bool) -> float:
    """Dense matrix-core peak for the main kernel's mix of work (TFLOP/s):
    with e4m3fn activations the residual product runs at the fp8 rate and
    the two low-rank products at the bf16 rate, so the peak is the work over
    the time each part needs at its own rate."""
    if not act8:
        return PEAK_BF16_TFLOPS
    M, K, N, r = w.M, w.in_features, w.out_features, w.rank
    f8, f16 = 2 * M * K * N, 2 * M * r * (K + N)
    return (f8 + f16) / (f8 / PEAK_FP8_TFLOPS + f16 / PEAK_BF16_TFLOPS)


# The sources that make up each kernel as launched: its own file, the
# shared device helpers and launch declarations, and the host code that
# chooses its variant and launch shape.
KERNEL_SOURCES = {
    "fused_kernel": ("tiled.hip", "device_common.hpp", "launch.hpp", "api.cpp"),
    "skinny_fullk_kernel": ("skinny.hip", "device_common.hpp", "launch.hpp", "api.cpp"),
    "skinny_kernel": ("skinny.hip", "device_common.hpp", "launch.hpp", "api.cpp"),
}


def source_digest(kernel: str | None = None) -> str:
    """sha256 over a kernel's sources (all of csrc/ without a kernel name): a
    counter record applies only to the sources it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_fp8_residual_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) if kernel else None
    files = [os.path.join(csrc, n) for n in names] if names else glob.glob(os.path.join(csrc, "*"))
    for f in sorted(files):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current sources of that kernel."""
    digest = source_digest(kernel)
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(f):
            if not line.startswith("traffic-record:"):
                continue
            try:
                rec = json.loads(line.split(":", 1)[1])
            except ValueError:
                continue
            if rec.get("kernel") == kernel and rec.get("workload") == workload and rec.get("sources") == digest:
                return rec
    return None


class Runner:
    """Rotating resident copies of one workload's inputs and a handle."""

    def __init__(self, w, args, dev, copies=0, act8=None):
        import torch

        from rank_fp8_residual_amd import Handle, Option, Path
        from rank_fp8_residual_amd import workloads as wl

        self.w = w
        t0 = time.time()
        self.d = wl.make_inputs(w, seed=args.seed)
        log(f"{w.name}: inputs drawn in {time.time() - t0:.1f}s")
        self.copies = copies or max(2, min(64, math.ceil(4 * MALL_BYTES / w.bytes)))
        self.sets = []
        for _ in range(self.copies):
            g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in self.d.items()}
            g["y"] = torch.empty((w.M, w.out_features), dtype=torch.bfloat16, device=dev)
            self.sets.append(g)
        torch.cuda.synchronize()
        self.h = Handle(dev.index)
        self.h.set_option(Option.PATH, {"auto": Path.AUTO, "skinny": Path.SKINNY, "tiled": Path.TILED}[args.path])
        self.h.set_option(Option.SPLIT_K, args.split_k)
        self.h.set_option(Option.T_SPLITS, args.t_splits)
        self.h.set_option(Option.T_LAUNCH, args.t_launch)
        self.act8 = args.act_fp8 if act8 is None else act8
        self.h.set_option(Option.ACT_FP8, int(self.act8))
        self.dev = dev

    def step(self, i):
        g = self.sets[i % self.copies]
        self.h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=g["y"])

    def ramp(self, ms):
        """Untimed steps for at least `ms` milliseconds of wall time, so that
        the clocks have ramped up under this load before anything is timed."""
        import torch

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(10):
                self.step(n)
                n += 1
            torch.cuda.synchronize()
        return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n}

    def timed(self, warmup, steps):
        """Warm up, then time exactly `steps` steps: ms per step."""
        import torch

        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(self.dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            self.step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def step_spread(self, steps):
        """p10 / p50 / p90 of single-step times (an event pair per step)."""
        import torch

        stream = torch.cuda.current_stream(self.dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            self.step(i)
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        q = lambda f: round(t[min(len(t) - 1, int(f * len(t)))] * 1e3, 2)
        return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "unit": "us"}

    def kernel_times(self, steps):
        """Average duration per launch of each kernel kind (library events)."""
        import torch

        from rank_fp8_residual_amd import Kernel, Option

        self.h.set_option(Option.PROFILE, 1)
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        kt = {}
        for name, kind in (("pad_a", Kernel.PAD_A), ("main", Kernel.MAIN), ("skinny", Kernel.SKINNY),
                           ("quant", Kernel.QUANT)):
            ms, n = self.h.kernel_time(kind, reset=True)
            if n:
                kt[name] = ms / n
        self.h.set_option(Option.PROFILE, 0)
        return kt

    def release(self):
        import torch

        self.sets = []
        torch.cuda.empty_cache()


def kernel_name(w, kind):
    """The kernel function behind a kernel kind on this workload.  The
    skinny kind has two: skinny_fullk_kernel takes up to 16 rows with
    2048 < in <= 8192, at least 192 groups of 32 output columns and at most
    that many T pieces (16 ranks x the K phases: 4 up to in = 4096, else 8),
    the library's automatic rule restated; skinny_kernel takes the rest."""
    if kind != "skinny":
        return KERNEL_NAMES[kind]
    groups = -(-w.out_features // 32)
    r_pad = -(-w.rank // 64) * 64 if w.rank else 0
    pieces = (r_pad // 16) * (4 if w.in_features <= 4096 else 8)
    fullk = w.M <= 16 and 2048 < w.in_features <= 8192 and groups >= 192 and pieces <= min(groups, 256)
    return "skinny_fullk_kernel" if fullk else "skinny_kernel"


def roofline(w, kt, ms_step, act8=False):
    """Roofline of the dominant kernel.  Its duration per launch is the timed
    region's time per step when the step launches that kernel alone (events
    bracketing back-to-back launches, as a profiler's trace sees them), else
    the library's per-launch event pairs."""
    dom = max(kt, key=kt.get)
    fl, by = kernel_flops_bytes(w, dom)
    dur_s = (ms_step if len(kt) == 1 else kt[dom]) * 1e-3
    peak = mfma_peak(w, act8 and dom == "main")
    if fl and fl / by > peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(fl / dur_s / 1e12, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s"}
        if act8 and dom == "main":
            roof["peak_note"] = "e4m3fn residual product at 5.0 PFLOP/s, bf16 low-rank products at 2.5 PFLOP/s"
    else:
        roof = {"bound": "hbm", "achieved": round(by / dur_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    kname = kernel_name(w, dom)
    rec = traffic_record(kname, w.name + ("+act_fp8" if act8 else ""))
    roof["traffic"] = rec["hbm_bytes"] if rec else None
    if rec:
        roof["traffic_detail"] = {k: rec[k] for k in ("fetch_bytes", "write_bytes", "scale", "profile") if k in rec}
    roof["kernel"] = kname
    roof["kernel_us"] = round(dur_s * 1e6, 2)
    roof["kernel_us_event_pairs"] = {k: round(v * 1e3, 2) for k, v in kt.items()}
    roof["algorithmic"] = {"flops": fl, "bytes": by}
    return roof


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} / WORLD_SIZE {world} is not supported "
              "(the forward's rows shard across GPUs with no communication, so N GPUs give N times "
              "the one-GPU figure)", file=sys.stderr)
        sys.exit(2)

    import torch

    from rank_fp8_residual_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    w = wl.WORKLOADS[args.workload]
    log("workload", w)
    run = Runner(w, args, dev, args.copies)
    log(f"{run.copies} rotating copies resident ({run.copies * w.bytes / 2**20:.0f} MiB)")

    clock_ramp = run.ramp(args.ramp_ms)
    log(f"clock ramp: {clock_ramp['steps']} untimed steps in {clock_ramp['ms']} ms")
    ms_step = run.timed(args.warmup, args.steps)
    tflops = w.flops / (ms_step * 1e-3) / 1e12
    gbs = w.bytes / (ms_step * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {ms_step * 1e3:.2f} us/step, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s")
    spread = run.step_spread(min(args.steps, 200))
    kt = run.kernel_times(args.steps)
    roof = roofline(w, kt, ms_step, run.act8)
    log("kernel us", roof["kernel_us"], "event pairs", roof["kernel_us_event_pairs"], "traffic", roof["traffic"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, run.d, run.sets[0], args.cpu_seconds)
    run.release()

    summary = None
    if not args.no_summary:
        summary = {}
        cases = [(name, False) for name in wl.WORKLOADS] + [(name, True) for name in ACT8_SUMMARY]
        for name, act8 in cases:
            if name == w.name and act8 == run.act8:
                continue
            wo = wl.WORKLOADS[name]
            r = Runner(wo, args, dev, act8=act8)
            steps = 20 if wo.flops > 1e12 else 100
            r.ramp(min(args.ramp_ms, 200.0))
            ms = r.timed(10 if wo.flops > 1e12 else 100, steps)
            k = r.kernel_times(steps)
            ro = roofline(wo, k, ms, act8)
            key = name + ("+act_fp8" if act8 else "")
            summary[key] = {
                "M": wo.M, "in": wo.in_features, "out": wo.out_features, "r": wo.rank,
                "activations": "e4m3fn" if act8 else "bf16",
                "us_per_step": round(ms * 1e3, 2),
                "TFLOP/s": round(wo.flops / (ms * 1e-3) / 1e12, 2),
                "GB/s": round(wo.bytes / (ms * 1e-3) / 1e9, 1),
                "kernel_us": {k2: round(v * 1e3, 2) for k2, v in k.items()},
                "roofline": {k2: ro[k2] for k2 in ("bound", "achieved", "peak", "unit", "frac", "kernel", "traffic")},
            }
            log(key, summary[key])
            r.release()

        for name in CONVERT_SUMMARY:
            key = "convert+" + name
            summary[key] = convert_timing(wl.WORKLOADS[name], dev)
            log(key, summary[key])
        for name in PAIR_SUMMARY:
            key = "pair+" + name
            summary[key] = pair_timing(wl.WORKLOADS[name], args, dev)
            log(key, summary[key])

    if args.copy_probe:
        copy_probe(dev)
    probe = None if args.no_read_probe else read_probe(dev)
    if probe and summary and "skinny" in summary:
        summary["skinny"]["vs_read_probe"] = round(probe["best"]["us"] / summary["skinny"]["us_per_step"], 4)
    if probe and w.name == "skinny" and not run.act8:
        roof["vs_read_probe"] = round(probe["best"]["us"] / (ms_step * 1e3), 4)

    line = {
        "metric": "fused LiteLinear TFLOP/s and HBM GB/s vs roofline, M=3630 in=2048 out=8192 r=64"
        if args.workload == HEADLINE else f"fused LiteLinear TFLOP/s and HBM GB/s vs roofline, {args.workload}",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3fn x e4m3fn residual, bf16 low-rank" if run.act8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: M={w.M} in={w.in_features} out={w.out_features} r={w.rank}; "
                        "x/A/B/bias bf16, Q e4m3fn with per-tensor scale, y bf16"
                        + ("; x quantised to e4m3fn per row for the residual product" if run.act8 else ""),
            "M": w.M, "in": w.in_features, "out": w.out_features, "r": w.rank,
            "rotating_copies": run.copies, "hbm_GBps": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "mfma_frac": round(tflops / mfma_peak(w, run.act8), 4),
            "flops_per_step": w.flops, "bytes_per_step": w.bytes,
            "step_us": spread,
        },
        "roofline": roof,
        "clock_ramp": clock_ramp,
        "hbm_read_probe": probe,
        "cpu_baseline": cpu,
        "device": device_info(dev),
        "workloads": summary,
    }
    print(json.dumps(line), flush=True)


def device_info(dev) -> dict:
    """Name, architecture, compute units and peak clocks of the device."""
    import ctypes

    import torch

    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count}
    from rank_fp8_residual_amd import litelinear as L

    try:
        # the HIP runtime the library itself is linked against (symbol lookup
        # through its handle searches its dependencies)
        get_attr = L.lib().hipDeviceGetAttribute
    except AttributeError:
        return info
    # hipDeviceAttributeClockRate and hipDeviceAttributeMemoryClockRate
    # (hip_runtime_api.h, ROCm 7), both in kHz
    for key, attr in (("peak_clock_mhz", 5), ("memory_clock_mhz", 60)):
        v = ctypes.c_int()
        if get_attr(ctypes.byref(v), attr, dev.index) == 0:
            info[key] = v.value // 1000
    return info


def pair_timing(w, args, dev, steps=100):
    """litelinear_forward_pair on two outputs of the workload's shape sharing
    x and B (a gate/up pair), against the same two outputs as two forwards."""
    import torch

    from rank_fp8_residual_amd import Handle
    from rank_fp8_residual_amd import workloads as wl

    d1 = wl.make_inputs(w, seed=args.seed)
    d2 = wl.make_inputs(w, seed=args.seed + 1)
    t = lambda v: v.to(dev) if isinstance(v, torch.Tensor) else v
    g1 = {k: t(v) for k, v in d1.items()}
    g2 = {k: t(v) for k, v in d2.items()}
    g2["x"], g2["B"] = g1["x"], g1["B"]
    y1 = torch.empty((w.M, w.out_features), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty_like(y1)
    h = Handle(dev.index)
    pair = lambda: h.forward_pair(g1["x"], g1["B"], (g1["A"], g1["Q"], g1["scale"], g1["bias"]),
                                  (g2["A"], g2["Q"], g2["scale"], g2["bias"]), out=(y1, y2))
    two = lambda: (h.forward(g1["x"], g1["A"], g1["B"], g1["Q"], g1["scale"], g1["bias"], out=y1),
                   h.forward(g2["x"], g2["A"], g2["B"], g2["Q"], g2["scale"], g2["bias"], out=y2))
    # Blocks of the two variants alternate, so that clock and power drift
    # over the run falls on both alike; each reports its median block.
    times = {"pair": [], "two_forwards": []}
    for _ in range(50):
        pair()
        two()
    torch.cuda.synchronize()
    block = max(1, steps // 10)
    for _ in range(10):
        for name, fn in (("pair", pair), ("two_forwards", two)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(block):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / block * 1e3)
    res = {k + "_us": round(statistics.median(v), 2) for k, v in times.items()}
    res["TFLOP/s_pair"] = round(2 * w.flops / (res["pair_us"] * 1e-6) / 1e12, 2)
    res["note"] = "two outputs of this shape sharing x and B; T computed once by the pair"
    return res


def convert_timing(w, dev, steps=20):
    """litelinear_residual_quantize on the workload's weight shapes (W [out, in]
    bf16, rank r): e4m3fn codes and scale of W - A B.  Both passes read W;
    algorithmic bytes count W, A, B once and the codes once."""
    import torch

    from rank_fp8_residual_amd import Handle

    out_f, in_f, r = w.out_features, w.in_features, w.rank
    nbytes = 2 * out_f * in_f + 2 * r * (out_f + in_f) + out_f * in_f
    copies = max(2, min(16, math.ceil(4 * MALL_BYTES / nbytes)))
    g = torch.Generator(device="cpu").manual_seed(7)
    sets = []
    for _ in range(copies):
        W = (torch.randn(out_f, in_f, generator=g) * 0.05).to(torch.bfloat16).to(dev)
        A = (torch.randn(out_f, r, generator=g) * 0.01).to(torch.bfloat16).to(dev)
        B = torch.randn(r, in_f, generator=g).to(torch.bfloat16).to(dev)
        codes = torch.empty((out_f, in_f), dtype=torch.uint8, device=dev)
        sets.append((W, A, B, codes))
    scale = torch.empty((1,), dtype=torch.float32, device=dev)
    h = Handle(dev.index)
    from rank_fp8_residual_amd import litelinear as L

    def step(i):
        W, A, B, codes = sets[i % copies]
        st = L.lib().litelinear_residual_quantize(h._h, W.data_ptr(), A.data_ptr(), B.data_ptr(), out_f, in_f, r,
                                                  codes.data_ptr(), scale.data_ptr(),
                                                  torch.cuda.current_stream(dev).cuda_stream)
        if st:
            raise RuntimeError(f"litelinear_residual_quantize: status {st}")

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2 * 2 * out_f * in_f * r  # A B in each of the two passes
    del sets
    torch.cuda.empty_cache()
    return {"out": out_f, "in": in_f, "r": r, "us_per_call": round(ms * 1e3, 2),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2), "algorithmic_bytes": nbytes}


READ_PROBE_BYTES = 64 << 20  # the skinny workload's residual codes (8192 x 8192 bytes)


def read_probe(dev, nbytes=READ_PROBE_BYTES, steps=60):
    """The chip's plain streaming-read rate for `nbytes`, the ceiling of a
    path that streams that much once: litelinear_read_probe over rotating
    copies (past the Infinity Cache), timed like a bench step (events around
    back-to-back launches), for a sweep of launch shapes; the best is the
    ceiling."""
    import torch

    from rank_fp8_residual_amd import Handle

    copies = max(2, math.ceil(4 * MALL_BYTES / nbytes))
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(i) for i in range(copies)]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    h = Handle(dev.index)
    results = []
    for wgs in (256, 512, 1024, 2048):
        for unroll in (4, 8, 16):
            for nt in (False, True):
                launch = lambda i: h.read_probe(bufs[i % copies], sink, wgs, unroll, nt)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                i = 0
                while (time.perf_counter() - t0) < 0.05 or i < 100:
                    launch(i)
                    i += 1
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for j in range(steps):
                    launch(j)
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / steps * 1e3
                results.append({"work_groups": wgs, "unroll": unroll, "nontemporal": nt, "us": round(us, 2),
                                "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)})
    best = min(results, key=lambda r: r["us"])
    del bufs
    torch.cuda.empty_cache()
    log(f"read probe ({nbytes >> 20} MiB, {copies} rotating copies): best {best}")
    return {"bytes": nbytes, "rotating_copies": copies, "best": best,
            "frac_of_peak": round(best["GB/s"] / PEAK_HBM_GBS, 4),
            "sweep": sorted(results, key=lambda r: r["us"])[:6]}


def copy_probe(dev, reps=5):
    """A plain device copy of COPY_PROBE_BYTES: under a counter run its
    FETCH_SIZE / WRITE_SIZE per dispatch give the scale of those counters
    (expected COPY_PROBE_BYTES each way)."""
    import torch

    src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {COPY_PROBE_BYTES} bytes")


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
