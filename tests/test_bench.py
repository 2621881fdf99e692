"""bench.py's accounting and output contract.

* CPU: the algorithmic flops and bytes the roofline is charged with match
  the per-workload figures tabulated for the method (three products counted
  once; every input read once and y written once), the mixed matrix-core
  peak of the e4m3fn-activation mode, and the refusal of more than one GPU.
* GPU: one short run prints one JSON line with every field the contract asks
  for (metric, value, roofline with bound / achieved / peak / unit / frac /
  traffic, cpu_baseline when asked, device).
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench
from rank_fp8_residual_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# GFLOP and MB of one forward, tabulated independently of the code that
# computes them (rounded as tabulated).
TABLE = {
    "tiny": (0.009437, 0.148),
    "skinny": (2.181, 69.75),
    "llm": (70.87, 51.39),
    "dit_r32": (124.2, 91.79),
    "dit_r64": (126.6, 92.45),
    "dit_r512": (159.9, 101.6),
    "large": (2543.0, 759.2),
}


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_work_matches_the_table(name):
    w = wl.WORKLOADS[name]
    gflop, mb = TABLE[name]
    fl, by = bench.kernel_flops_bytes(w, "main")
    assert abs(fl / 1e9 - gflop) <= 0.0006 * gflop + 1e-6, (fl / 1e9, gflop)
    assert abs(by / 1e6 - mb) <= 0.0006 * mb + 1e-3, (by / 1e6, mb)


def test_mixed_peak_of_the_fp8_activation_mode():
    # 4.82 PFLOP/s on DiT r64 and 4.40 on Large: the residual product at the
    # e4m3fn rate (5.0), the low-rank products at the bf16 rate (2.5)
    assert bench.mfma_peak(wl.WORKLOADS["dit_r64"], False) == bench.PEAK_BF16_TFLOPS
    assert abs(bench.mfma_peak(wl.WORKLOADS["dit_r64"], True) - 4818.8) < 0.1
    assert abs(bench.mfma_peak(wl.WORKLOADS["large"], True) - 4404.8) < 0.1
    for w in wl.WORKLOADS.values():
        assert bench.PEAK_BF16_TFLOPS < bench.mfma_peak(w, True) <= bench.PEAK_FP8_TFLOPS


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


@pytest.mark.gpu
def test_bench_json_line(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] bench json line (tiny, 5 steps)", file=sys.stderr, flush=True)
    p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "5",
                        "--warmup", "5", "--no-summary", "--no-cpu-baseline", "--ramp-ms", "50"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "device"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5 and d["value"] > 0
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"].startswith("tiny")
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma", "alu") and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert d["device"]["compute_units"] > 0
    assert d["clock_ramp"]["ms"] >= 50 and d["clock_ramp"]["steps"] > 0
    probe = d["hbm_read_probe"]
    assert probe["bytes"] == 64 << 20 and 0 < probe["best"]["GB/s"] < 8000


def test_kernel_name_follows_the_skinny_rule():
    """The skinny workload runs the all-of-K kernel; other skinny shapes
    (more rows, narrow outputs, short or long K) the K-sliced one."""
    import bench
    from rank_fp8_residual_amd import workloads as wl
    assert bench.kernel_name(wl.WORKLOADS["skinny"], "skinny") == "skinny_fullk_kernel"
    assert bench.kernel_name(wl.WORKLOADS["dit_r64"], "main") == "fused_kernel"
    import dataclasses
    W = wl.WORKLOADS["skinny"]
    for kw in ({"M": 17}, {"out_features": 4096}, {"in_features": 2048}, {"in_features": 16384}):
        assert bench.kernel_name(dataclasses.replace(W, **kw), "skinny") == "skinny_kernel", kw


def test_kernel_sources_exist():
    """Every file a traffic record's digest covers is a library source."""
    import bench
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "rank_fp8_residual_amd", "csrc")
    for kernel, names in bench.KERNEL_SOURCES.items():
        for n in names:
            assert os.path.isfile(os.path.join(csrc, n)), (kernel, n)
        assert bench.source_digest(kernel) != bench.source_digest()
