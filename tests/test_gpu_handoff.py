"""The hand-over of T = x B^T between work-groups of one launch.

* Graph capture: a forward captured into a graph and replayed with new input
  values (copied into the captured tensors between replays, with other eager
  work and synchronisations in between) matches the oracle on every replay.
  The counters start each launch at zero, so nothing in the capture is stale.
* The bounded waits report when they give up: a test hook makes every wait
  look for one count more than the launch produces and give up after a few
  polls (all kernels still end normally); the error then surfaces as
  LITELINEAR_ERR_SYNC, once, and the handle works normally afterwards.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Handle, LiteLinearError, Option, Path, Status
from rank_fp8_residual_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def to_dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def oracle_y(d):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"], d["scale"],
                          d["bias"])


# (M, in, out, r, path, act8): the tiled kernel with T producers (64- and
# 256-column T blocks, K-sliced T), the skinny kernels (K-sliced, and all of
# K per work-group), the fp8-activation mode
CAPTURE_CASES = [
    (1024, 512, 2048, 64, Path.TILED, False),
    (600, 1024, 1024, 256, Path.TILED, False),
    (300, 1280, 520, 80, Path.TILED, False),
    (16, 2048, 4096, 64, Path.SKINNY, False),
    (16, 4096, 8192, 64, Path.SKINNY, False),
    (1024, 512, 2048, 64, Path.TILED, True),
]


@pytest.mark.parametrize("case", CAPTURE_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4].name}"
                         + ("-act8" if c[5] else ""))
def test_graph_capture_replays_with_new_inputs(dev, case):
    M, K, N, r, path, act8 = case
    d0 = wl.random_inputs(M, K, N, r, seed=500)
    g = to_dev(d0, dev)
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(path))
    h.set_option(Option.ACT_FP8, int(act8))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("capture", case, "eager warm-up")
    h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=y)
    torch.cuda.synchronize()
    other = Handle(dev.index)
    for rep, seed in enumerate((501, 502, 503)):
        d = wl.random_inputs(M, K, N, r, seed=seed)
        d["scale"] = d0["scale"]  # the scale is a launch argument, fixed at capture
        for k in ("x", "A", "B", "Q", "bias"):
            g[k].copy_(d[k])
        torch.cuda.synchronize()
        say("capture", case, "replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], act_fp8=act8)
        parity.check(parity.to_f64(y), y_ref, False)
        # eager work of the program between replays, on another handle
        ye = other.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
        torch.cuda.synchronize()
        parity.check(parity.to_f64(ye), oracle_y(d), False)
    del graph


def test_capture_refuses_to_grow_the_workspace(dev):
    """A call under capture whose shape needs more workspace than the handle
    holds is refused (UNSUPPORTED), and the capture itself stays intact."""
    d = wl.random_inputs(512, 512, 1024, 64, seed=510)
    g = to_dev(d, dev)
    h = Handle(dev.index)
    say("capture refuses growth")
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(LiteLinearError) as ei:
        with torch.cuda.graph(graph):
            h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert ei.value.status == Status.UNSUPPORTED
    torch.cuda.synchronize()
    y = h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    parity.check(parity.to_f64(y), oracle_y(d), False)


# (M, in, out, r, path): producers with one and with several K slices,
# 256-column T blocks, a pair, the skinny kernels (one and several slices,
# all of K per work-group)
TIMEOUT_CASES = [
    (1024, 512, 2048, 64, Path.TILED), (300, 1280, 520, 80, Path.TILED), (600, 1024, 1024, 256, Path.TILED),
    (16, 2048, 4096, 64, Path.SKINNY), (40, 512, 640, 32, Path.SKINNY),
    (16, 4096, 8192, 64, Path.SKINNY),
]


@pytest.mark.parametrize("case", TIMEOUT_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4].name}")
def test_wait_timeout_is_reported(dev, case):
    M, K, N, r, path = case
    d = wl.random_inputs(M, K, N, r, seed=520)
    g = to_dev(d, dev)
    y_ref = oracle_y(d)
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(path))
    assert h.device_status() == Status.OK
    say("timeout", case, "forced")
    h.set_option(Option.TEST_WAIT_TIMEOUT, 64)
    h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])  # queued normally
    torch.cuda.synchronize()
    h.set_option(Option.TEST_WAIT_TIMEOUT, 0)
    # the next call reports it instead of running ...
    with pytest.raises(LiteLinearError) as ei:
        h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert ei.value.status == Status.SYNC
    assert h.device_status() == Status.OK  # ... once
    # ... and the handle works again (its counters were reset)
    for _ in range(2):
        y = h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
        torch.cuda.synchronize()
        parity.check(parity.to_f64(y), y_ref, False)
    # the query reports it too
    say("timeout", case, "forced, query")
    h.set_option(Option.TEST_WAIT_TIMEOUT, 16)
    h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    h.set_option(Option.TEST_WAIT_TIMEOUT, 0)
    assert h.device_status() == Status.SYNC
    assert h.device_status() == Status.OK
    y = h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    parity.check(parity.to_f64(y), y_ref, False)


def test_no_timeout_in_normal_runs(dev):
    """Many launches of every T hand-over variant leave the error word clear."""
    h = Handle(dev.index)
    for M, K, N, r, path in TIMEOUT_CASES:
        d = wl.random_inputs(M, K, N, r, seed=530)
        g = to_dev(d, dev)
        h.set_option(Option.PATH, int(path))
        say("no timeout", (M, K, N, r, path.name))
        for _ in range(20):
            y = h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
        torch.cuda.synchronize()
        assert h.device_status() == Status.OK
        parity.check(parity.to_f64(y), oracle_y(d), False)


def test_pair_back_to_back_with_new_inputs(dev):
    """Two shared-B pairs with different inputs queued back to back on one
    handle (T computed once per pair, consumers of both outputs counted)."""
    h = Handle(dev.index)
    outs = []
    for seed in (540, 541):
        d1 = wl.random_inputs(1024, 512, 2048, 64, seed=seed)
        d2 = wl.random_inputs(1024, 512, 1536, 64, seed=seed + 100)
        d2["x"], d2["B"] = d1["x"], d1["B"]
        g1, g2 = to_dev(d1, dev), to_dev(d2, dev)
        y1, y2 = h.forward_pair(g1["x"], g1["B"], (g1["A"], g1["Q"], g1["scale"], g1["bias"]),
                                (g2["A"], g2["Q"], g2["scale"], g2["bias"]))
        outs.append((d1, d2, y1, y2))
    torch.cuda.synchronize()
    say("pair back to back")
    for d1, d2, y1, y2 in outs:
        parity.check(parity.to_f64(y1), oracle_y(d1), False)
        parity.check(parity.to_f64(y2), oracle_y(d2), False)
