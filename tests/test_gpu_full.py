"""Full-size workloads, whole outputs, against the float64 CPU oracle.

Every workload runs in the launch configuration the bench times (the
automatic path, one handle), with two different input sets (seeds 0 and 1)
queued back to back on the same handle with no synchronisation between them.
Both outputs are compared element by element with the oracle over all rows:
a launch that read the T' blocks, T pieces, slice partials or counters of
the launch before it would produce the other seed's numbers and fail.

The fp8-activation mode is checked the same way against the oracle's
fp8-activation forward (whole output for seed 0, sampled rows for seed 1),
together with the method's own distance from the exact forward.  Gates are
in tests/parity.py; the float32-output mode must pass the literal max gate.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Handle, Option, Path
from rank_fp8_residual_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu

ACT8_MAX_RMS = 0.25
ACT8_REL_L1 = 4e-2


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


_inputs: dict = {}


def inputs(name: str, seed: int) -> dict:
    """Seeded CPU inputs of a workload, kept for the module (both modes)."""
    key = (name, seed)
    if key not in _inputs:
        if len(_inputs) >= 4:
            _inputs.pop(next(iter(_inputs)))
        _inputs[key] = wl.make_inputs(wl.WORKLOADS[name], seed=seed)
    return _inputs[key]


def to_dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def fwd(h, g):
    return h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"])


def ref_rows(d, act8=False):
    return lambda rows: oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"],
                                       d["scale"], d["bias"], rows=rows, act_fp8=act8)


def sample_rows(M, n=48):
    return np.unique(np.concatenate([np.linspace(0, M - 1, n).astype(np.int64), [0, M - 1, max(M - 7, 0)]]))


def short(m):
    return {k: (round(v, 6) if isinstance(v, float) else v) for k, v in m.items()}


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_workload_full_output_two_inputs_back_to_back(dev, name):
    w = wl.WORKLOADS[name]
    d0, d1 = inputs(name, 0), inputs(name, 1)
    g0, g1 = to_dev(d0, dev), to_dev(d1, dev)
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(Path.AUTO))
    say("full", name, w, "seeds 0 and 1 back to back")
    y0 = fwd(h, g0)
    y1 = fwd(h, g1)  # queued right behind the first, same handle, no sync
    h32 = Handle(dev.index)
    h32.set_option(Option.OUTPUT_F32, 1)
    y0f = fwd(h32, g0)
    torch.cuda.synchronize()
    del g0, g1
    say("full", name, "oracle seed 0")
    m0 = parity.check_full(y0, ref_rows(d0), w.M, False)
    say("full", name, "seed 0", short(m0))
    m0f = parity.check_full(y0f, ref_rows(d0), w.M, True)
    say("full", name, "seed 0 float32 output", short(m0f))
    del y0, y0f
    say("full", name, "oracle seed 1")
    m1 = parity.check_full(y1, ref_rows(d1), w.M, False)
    say("full", name, "seed 1", short(m1))
    del y1
    torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_workload_full_output_act8(dev, name):
    w = wl.WORKLOADS[name]
    d0, d1 = inputs(name, 0), inputs(name, 1)
    g0, g1 = to_dev(d0, dev), to_dev(d1, dev)
    h = Handle(dev.index)
    h.set_option(Option.ACT_FP8, 1)
    say("full act8", name, w, "seeds 0 and 1 back to back")
    y0 = fwd(h, g0)
    y1 = fwd(h, g1)
    torch.cuda.synchronize()
    del g0, g1
    m0 = parity.check_full(y0, ref_rows(d0, act8=True), w.M, False)
    say("full act8", name, "seed 0", short(m0))
    rows = np.arange(w.M) if w.M <= 64 else sample_rows(w.M)
    ridx = torch.from_numpy(rows).to(dev)
    ys1 = parity.to_f64(y1[ridx])
    parity.check(ys1, ref_rows(d1, act8=True)(rows), False)
    # the method's own error: fp8 activations against the exact forward
    ys0 = parity.to_f64(y0[ridx])
    y_exact = ref_rows(d0)(rows)
    e = parity.metrics(ys0, y_exact)
    say("act8 vs exact", name, short(e))
    assert e["rel_l1"] <= ACT8_REL_L1, e
    assert np.all(np.abs(ys0 - y_exact) <= ACT8_MAX_RMS * e["rms"] + parity.half_ulp_bf16(y_exact)), e
    del y0, y1
    torch.cuda.empty_cache()
