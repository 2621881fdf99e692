"""litelinear_forward_noalloc: the forward with its workspace carved out of
the library's fixed per-device scratch instead of allocated memory.

Through the C ABI, two calls in a row on one handle (the second with a
smaller input) must equal litelinear_forward's outputs bit for bit (the same
kernels, on the same inputs) and meet the oracle's gates; a call that needs
more than the scratch holds is refused with LITELINEAR_ERR_SCRATCH before
anything is queued; the call can be captured into a graph and replayed.
"""
from __future__ import annotations

import sys

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


def fwd(h, g, noalloc):
    return h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"],
                     noalloc=noalloc)


# pairs of calls in a row, the second smaller: (M, in, out, r) x 2 and options
CASES = [
    ("dit", (3630, 2048, 8192, 64), (1000, 2048, 8192, 64), {}),
    ("llm", (2048, 4096, 4096, 64), (700, 4096, 2048, 64), {}),
    ("skinny", (16, 8192, 8192, 64), (9, 4096, 4096, 32), {}),
    ("tiny", (64, 256, 256, 16), (40, 256, 128, 8), {}),
    ("wide-T", (4096, 512, 4096, 256), (1024, 512, 4096, 256), {}),
    ("act8", (3630, 2048, 8192, 64), (2000, 2048, 4096, 64), {Option.ACT_FP8: 1}),
    ("pad-A", (700, 512, 1024, 20), (300, 512, 512, 12), {}),
    ("f32-out", (2048, 1024, 2048, 64), (16, 1024, 2048, 64), {Option.OUTPUT_F32: 1}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_noalloc_matches_forward_two_calls(dev, case):
    name, big, small, opts = case
    h_ref, h_na = Handle(dev.index), Handle(dev.index)
    for k, v in opts.items():
        h_ref.set_option(k, v)
        h_na.set_option(k, v)
    act8 = bool(opts.get(Option.ACT_FP8, 0))
    out_f32 = bool(opts.get(Option.OUTPUT_F32, 0))
    for i, shape in enumerate((big, small)):
        M, K, N, r = shape
        d = wl.random_inputs(M, K, N, r, seed=800 + i)
        g = to_dev(d, dev)
        say("noalloc", name, i, shape)
        y_na = fwd(h_na, g, True)
        y_ref = fwd(h_ref, g, False)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ref), (name, shape)
        rows = torch.arange(M) if M <= 256 else torch.linspace(0, M - 1, 200).long().unique()
        yo = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows.numpy(), act_fp8=act8)
        parity.check(parity.to_f64(y_na[rows.to(dev)]), yo, out_f32)


def test_noalloc_refuses_what_does_not_fit(dev):
    """The 16384 x 4096 e4m3fn-activation forward needs 64 MiB of activation
    codes: refused before anything is queued; a fitting call then works."""
    h = Handle(dev.index)
    h.set_option(Option.ACT_FP8, 1)
    M, K, N, r = 16384, 4096, 256, 16
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    A = torch.zeros((N, r), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((r, K), dtype=torch.bfloat16, device=dev)
    Q = torch.zeros((N, K), dtype=torch.uint8, device=dev)
    say("noalloc too large")
    with pytest.raises(LiteLinearError) as ei:
        h.forward(x, A, B, Q, 1.0, None, noalloc=True)
    assert ei.value.status == Status.SCRATCH
    d = wl.random_inputs(512, 1024, 1024, 64, seed=810)
    g = to_dev(d, dev)
    y = fwd(h, g, True)
    torch.cuda.synchronize()
    parity.check(parity.to_f64(y), oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"],
                                                  act_fp8=True), False)


def test_noalloc_graph_capture(dev):
    """Captured and replayed with new inputs (no allocation in the capture)."""
    M, K, N, r = 1024, 512, 2048, 64
    d0 = wl.random_inputs(M, K, N, r, seed=820)
    g = to_dev(d0, dev)
    h = Handle(dev.index)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    graph = torch.cuda.CUDAGraph()
    say("noalloc capture")
    with torch.cuda.graph(graph):
        h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=y, noalloc=True)
    torch.cuda.synchronize()
    for seed in (821, 822):
        d = wl.random_inputs(M, K, N, r, seed=seed)
        d["scale"] = d0["scale"]
        for k in ("x", "A", "B", "Q", "bias"):
            g[k].copy_(d[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        parity.check(parity.to_f64(y), oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"]), False)
        # eager work between replays: the same entry point on another handle
        y2 = fwd(Handle(dev.index), g, True)
        torch.cuda.synchronize()
        assert torch.equal(y2, y)
