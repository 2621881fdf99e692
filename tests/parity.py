"""Parity gates shared by the GPU tests and the bench.

Tolerance (stated for the bf16 forward; the pages fix none):
  * mean relative error, read as relative L1:  sum|y - y_ref| / sum|y_ref| <= 5e-3
    (a per-element mean of |dy|/|y_ref| has no finite expectation when y_ref
    has a density at zero, so it is reported only);
  * max error against the float64 oracle:
      - float32 output:  max|y - y_ref| <= 2e-2 * RMS(y_ref)        (literal)
      - bf16 output:     |y - y_ref| <= 2e-2 * RMS(y_ref) + ulp_bf16(y_ref)/2
        element-wise; the half-ulp is the rounding of the exact value to the
        nearest bf16, which alone exceeds 2e-2 * RMS on the DiT workloads
        (outlier channels put |y| up to ~7 RMS).
The literal max/RMS figure is reported in every case.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L1_GATE = 5e-3
MAX_RMS_GATE = 2e-2


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), np.ldexp(1.0, -134))


def to_f64(y: torch.Tensor) -> np.ndarray:
    return y.detach().to("cpu").to(torch.float64).numpy()


def bf16_of(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float64 values to bf16, back in float64."""
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(torch.float64).numpy()


def metrics(y: np.ndarray, y_ref: np.ndarray) -> dict:
    d = np.abs(y - y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    l1 = float(np.sum(np.abs(y_ref)))
    nz = np.abs(y_ref) > 0
    return {
        "rms": rms,
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_over_rms": float(d.max() / rms) if d.size and rms > 0 else 0.0,
        "rel_l1": float(d.sum() / l1) if l1 > 0 else float(d.sum()),
        "mean_rel_elem": float(np.mean(d[nz] / np.abs(y_ref[nz]))) if nz.any() else 0.0,
        "finite": bool(np.all(np.isfinite(y))),
    }


def check(y: np.ndarray, y_ref: np.ndarray, out_f32: bool, rms: float | None = None) -> dict:
    """Assert the gates; ``rms`` overrides RMS(y_ref) (e.g. from a row sample)."""
    m = metrics(y, y_ref)
    r = m["rms"] if rms is None else rms
    assert m["finite"], "non-finite output"
    assert m["rel_l1"] <= REL_L1_GATE, m
    bound = MAX_RMS_GATE * r
    if not out_f32:
        bound = bound + half_ulp_bf16(y_ref)
    bad = np.abs(y - y_ref) > bound
    assert not bad.any(), {**m, "n_bad": int(bad.sum()), "first_bad": np.argwhere(bad)[:3].tolist()}
    return m


def check_full(y_dev: torch.Tensor, ref_rows, M: int, out_f32: bool, chunk: int = 1024) -> dict:
    """The gates of ``check`` on the whole output of a full-size call.

    ``ref_rows(rows)`` returns the float64 oracle output for an array of row
    indices; it is called chunk by chunk, the reference is kept whole (the
    max gate needs RMS over all of it), and the device output is converted
    to float64 one chunk at a time."""
    N = y_dev.shape[-1]
    y_ref = np.empty((M, N), np.float64)
    for m0 in range(0, M, chunk):
        y_ref[m0:m0 + chunk] = ref_rows(np.arange(m0, min(M, m0 + chunk), dtype=np.int64))
    rms = float(np.sqrt(np.mean(np.square(y_ref)))) if y_ref.size else 0.0
    sum_abs_ref, sum_abs_d, max_d, n_bad, first_bad = 0.0, 0.0, 0.0, 0, None
    finite = True
    for m0 in range(0, M, chunk):
        yr = y_ref[m0:m0 + chunk]
        y = to_f64(y_dev[m0:m0 + chunk])
        finite = finite and bool(np.all(np.isfinite(y)))
        d = np.abs(y - yr)
        sum_abs_ref += float(np.sum(np.abs(yr)))
        sum_abs_d += float(np.sum(d))
        max_d = max(max_d, float(d.max()) if d.size else 0.0)
        bound = MAX_RMS_GATE * rms
        if not out_f32:
            bound = bound + half_ulp_bf16(yr)
        bad = d > bound
        if bad.any():
            n_bad += int(bad.sum())
            if first_bad is None:
                i, j = np.argwhere(bad)[0]
                first_bad = [int(m0 + i), int(j), float(y[i, j]), float(yr[i, j])]
    m = {"rms": rms, "max_abs": max_d, "max_over_rms": max_d / rms if rms > 0 else 0.0,
         "rel_l1": sum_abs_d / sum_abs_ref if sum_abs_ref > 0 else sum_abs_d, "finite": finite,
         "n_bad": n_bad, "first_bad": first_bad, "rows": M}
    assert finite, m
    assert m["rel_l1"] <= REL_L1_GATE, m
    assert n_bad == 0, m
    return m
