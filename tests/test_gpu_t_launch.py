"""The tiled path with T = x B^T computed by a launch of its own (t_kernel),
queued ahead of the output tiles, instead of producer work-groups inside
their launch (LITELINEAR_OPT_T_LAUNCH).

* Forced on (2) for shapes of one and of up to eight K slices, ranks of one
  and two 64-rank blocks, ragged rows and ranks, both outputs, the
  fp8-activation mode, e4m3fnuz codes and the gated epilogue: full output
  against the float64 oracle.
* Exact-arithmetic inputs: both ways of computing T give the oracle's values
  bit for bit.
* Two calls with different inputs queued back to back on one handle (a
  consumer that read the other call's T' would fail), graph capture with
  replays on new inputs, a pair, and the bounded wait's error report.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Activation, Handle, LiteLinearError, Option, Path, Status
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


def handle(dev, t_launch, out_f32=False):
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(Path.TILED))
    h.set_option(Option.T_LAUNCH, t_launch)
    h.set_option(Option.OUTPUT_F32, int(out_f32))
    return h


def fwd(h, g, out=None):
    return h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=out)


def oracle_y(d, **kw):
    return oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], **kw)


# M, in, out, r: K slices of t_kernel = in / 1024 (r <= 64) or in / 512
# (64 < r <= 128), rounded up
SHAPES = [
    (2048, 4096, 4096, 64),   # the LLM grid (chosen automatically there), 4 slices
    (300, 1280, 520, 80),     # 128-rank blocks (r_pad 128), 3 slices, ragged
    (1000, 8192, 1024, 64),   # 8 slices
    (77, 4096, 900, 128),     # r_pad 128 at its largest in: 8 slices
    (513, 1008, 1000, 5),     # one slice, rank 5, ragged rows
    (4000, 512, 700, 33),     # 192 tiles of 128 x 128, ragged rank
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_t_launch_parity(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=7000 + M + r)
    g = to_dev(d, dev)
    say("t launch", shape, out_f32)
    y = fwd(handle(dev, 2, out_f32), g)
    torch.cuda.synchronize()
    parity.check(parity.to_f64(y), oracle_y(d), out_f32)


@pytest.mark.parametrize("shape", [(2048, 4096, 4096, 64), (300, 1280, 520, 80), (77, 4096, 900, 128),
                                   (513, 1008, 1000, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_t_launch_exact_bitwise(dev, shape):
    """Exact inputs: T' from its own launch, T' from in-launch producers and
    the oracle agree bit for bit (rank 1 here: with random inputs the one
    rank's bf16 rounding of T alone can reach the float32-output gate)."""
    M, K, N, r = shape
    d = wl.exact_inputs(M, K, N, r, seed=7100 + r)
    g = to_dev(d, dev)
    expect = parity.bf16_of(oracle_y(d))
    say("t launch exact", shape)
    for mode in (1, 2):
        y = parity.to_f64(fwd(handle(dev, mode), g))
        bad = np.argwhere(y != expect)
        assert bad.size == 0, (mode, bad[:5].tolist())


def test_t_launch_back_to_back_new_inputs(dev):
    """Two calls with different inputs queued on one handle without a
    synchronisation in between, then one call again: each matches the oracle
    on its own inputs."""
    M, K, N, r = 2048, 4096, 4096, 64
    h = handle(dev, 0)  # chosen automatically on this grid
    ds = [wl.random_inputs(M, K, N, r, seed=s) for s in (7200, 7201, 7202)]
    gs = [to_dev(d, dev) for d in ds]
    say("t launch back to back")
    ys = [fwd(h, g) for g in gs]
    torch.cuda.synchronize()
    for d, y in zip(ds, ys):
        parity.check_full(y, lambda rows, d=d: oracle_y(d, rows=rows), M, False)


VARIANTS = [
    ("act8", dict(act8=True)),
    ("fnuz", dict(fnuz=True)),
    ("geglu", dict(act=Activation.GEGLU)),
    ("gelu", dict(act=Activation.GELU_TANH)),
]


@pytest.mark.parametrize("name,opts", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_t_launch_variants(dev, name, opts):
    M, K, N, r = 1024, 2048, 2048, 64
    fnuz = opts.get("fnuz", False)
    d = wl.random_inputs(M, K, N, r, seed=7300, q_format="e4m3fnuz" if fnuz else "e4m3fn")
    g = to_dev(d, dev)
    h = handle(dev, 2)
    h.set_option(Option.ACT_FP8, int(opts.get("act8", False)))
    h.set_option(Option.Q_FORMAT, int(fnuz))
    act = opts.get("act", Activation.NONE)
    h.set_option(Option.ACTIVATION, int(act))
    say("t launch variant", name)
    y = parity.to_f64(fwd(h, g))
    torch.cuda.synchronize()
    v_ref = oracle_y(d, act_fp8=opts.get("act8", False), q_format="e4m3fnuz" if fnuz else "e4m3fn")
    if act == Activation.GEGLU:
        from tests.test_gpu_variants import check_geglu
        check_geglu(y, v_ref, False)
    elif act == Activation.GELU_TANH:
        y_ref = oracle.gelu_tanh(v_ref)
        rms = float(np.sqrt(np.mean(v_ref ** 2)))
        assert np.all(np.abs(y - y_ref) <= 1.13 * parity.MAX_RMS_GATE * rms + parity.half_ulp_bf16(y_ref))
    else:
        parity.check(y, v_ref, False)


def test_t_launch_pair(dev):
    """A shared-B pair whose T comes from its own launch (both T' written by
    it), two pairs with different inputs back to back."""
    h = handle(dev, 2)
    outs = []
    for seed in (7400, 7401):
        d1 = wl.random_inputs(1024, 2048, 2048, 64, seed=seed)
        d2 = wl.random_inputs(1024, 2048, 1536, 64, seed=seed + 100)
        d2["x"], d2["B"] = d1["x"], d1["B"]
        g1, g2 = to_dev(d1, dev), to_dev(d2, dev)
        y1, y2 = h.forward_pair(g1["x"], g1["B"], (g1["A"], g1["Q"], g1["scale"], g1["bias"]),
                                (g2["A"], g2["Q"], g2["scale"], g2["bias"]))
        outs.append((d1, d2, y1, y2))
    torch.cuda.synchronize()
    say("t launch pair")
    for d1, d2, y1, y2 in outs:
        parity.check(parity.to_f64(y1), oracle_y(d1), False)
        parity.check(parity.to_f64(y2), oracle_y(d2), False)


@pytest.mark.parametrize("act8", [False, True], ids=["bf16", "act8"])
def test_t_launch_graph_capture(dev, act8):
    """Captured with the T launch, replayed on new inputs with eager work in
    between: every replay matches the oracle, with bf16 and with e4m3fn
    activations (the quantiser, the T launch and the output tiles)."""
    M, K, N, r = 1024, 2048, 2048, 64
    d0 = wl.random_inputs(M, K, N, r, seed=7500)
    g = to_dev(d0, dev)
    h = handle(dev, 2)
    h.set_option(Option.ACT_FP8, int(act8))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("t launch capture", "act8" if act8 else "bf16")
    fwd(h, g, out=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(h, g, out=y)
    torch.cuda.synchronize()
    other = handle(dev, 2)
    other.set_option(Option.ACT_FP8, int(act8))
    for seed in (7501, 7502, 7503):
        d = wl.random_inputs(M, K, N, r, seed=seed)
        d["scale"] = d0["scale"]
        for k in ("x", "A", "B", "Q", "bias"):
            g[k].copy_(d[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_ref = oracle_y(d, act_fp8=act8)
        parity.check(parity.to_f64(y), y_ref, False)
        ye = fwd(other, g)
        torch.cuda.synchronize()
        parity.check(parity.to_f64(ye), y_ref, False)
    del graph


def test_t_launch_wait_timeout_is_reported(dev):
    """The output tiles' bounded wait for T' still reports giving up (test
    hook), and the handle works again afterwards."""
    M, K, N, r = 1024, 2048, 2048, 64
    d = wl.random_inputs(M, K, N, r, seed=7600)
    g = to_dev(d, dev)
    h = handle(dev, 2)
    say("t launch timeout")
    h.set_option(Option.TEST_WAIT_TIMEOUT, 64)
    fwd(h, g)
    torch.cuda.synchronize()
    h.set_option(Option.TEST_WAIT_TIMEOUT, 0)
    with pytest.raises(LiteLinearError) as ei:
        fwd(h, g)
    assert ei.value.status == Status.SYNC
    for _ in range(2):
        y = fwd(h, g)
        torch.cuda.synchronize()
        parity.check(parity.to_f64(y), oracle_y(d), False)
    assert h.device_status() == Status.OK
