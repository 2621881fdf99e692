"""GPU parity of the stream kernel (LITELINEAR_OPT_PATH = 3; the automatic
choice for M <= 16 with at least 128 work-groups of 32 output columns)
against the float64 oracle: ragged rows, columns, K and ranks, every rank
group count, the output and activation options, e4m3fnuz codes, and
repeat calls bit for bit (the T pieces are summed in a fixed order)."""
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


def handle(dev, path=Path.STREAM, opts=None):
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(path))
    for k, v in (opts or {}).items():
        h.set_option(k, v)
    return h


def fwd(h, g):
    y = h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    return y


STREAM_SHAPES = [  # M, in, out, r
    (16, 8192, 8192, 64), (1, 4096, 4096, 64), (5, 2048, 4104, 20), (16, 1008, 4096, 0), (9, 512, 8200, 200),
    (16, 4096, 4096, 512), (12, 16, 4096, 8), (16, 3072, 16384, 128),
]


@pytest.mark.parametrize("shape", STREAM_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_stream_parity(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=900 + M + r)
    say("stream", shape, "f32" if out_f32 else "bf16")
    h = handle(dev, opts={Option.OUTPUT_F32: int(out_f32)})
    g = to_dev(d, dev)
    y1 = fwd(h, g)
    y2 = fwd(h, g)
    assert torch.equal(y1, y2)
    parity.check(parity.to_f64(y1), oracle.forward(d["x"], d["A"] if r else None, d["B"] if r else None, d["Q"],
                                                   d["scale"], d["bias"]), out_f32)


def test_stream_is_the_automatic_choice_for_the_skinny_workload(dev):
    """The automatic path and the stream path give the same bits."""
    d = wl.random_inputs(16, 4096, 8192, 64, seed=910)
    g = to_dev(d, dev)
    say("stream auto")
    assert torch.equal(fwd(handle(dev, Path.AUTO), g), fwd(handle(dev, Path.STREAM), g))


@pytest.mark.parametrize("variant", ["gelu", "geglu", "fnuz", "fnuz-geglu"])
def test_stream_variants(dev, variant):
    fnuz = variant.startswith("fnuz")
    M, K, N, r = 13, 2048, 8192, 64
    d = wl.random_inputs(M, K, N, r, seed=920, q_format="e4m3fnuz" if fnuz else "e4m3fn")
    opts = {Option.Q_FORMAT: int(fnuz)}
    if variant == "gelu":
        opts[Option.ACTIVATION] = int(Activation.GELU_TANH)
    if variant.endswith("geglu"):
        opts[Option.ACTIVATION] = int(Activation.GEGLU)
    say("stream variant", variant)
    y = parity.to_f64(fwd(handle(dev, opts=opts), to_dev(d, dev)))
    v_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"],
                           q_format="e4m3fnuz" if fnuz else "e4m3fn")
    if variant == "gelu":
        y_ref = oracle.gelu_tanh(v_ref)
        rms = float(np.sqrt(np.mean(v_ref ** 2)))
        assert np.all(np.abs(y - y_ref) <= 1.13 * parity.MAX_RMS_GATE * rms + parity.half_ulp_bf16(y_ref))
    elif variant.endswith("geglu"):
        from tests.test_gpu_variants import check_geglu
        assert y.shape == (M, N // 2)
        check_geglu(y, v_ref, False)
    else:
        parity.check(y, v_ref, False)


def test_stream_refuses_shapes_it_does_not_take(dev):
    d = wl.random_inputs(17, 1024, 8192, 64, seed=930)  # more than 16 rows
    g = to_dev(d, dev)
    with pytest.raises(LiteLinearError) as ei:
        handle(dev).forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert ei.value.status == Status.UNSUPPORTED
    d = wl.random_inputs(16, 1024, 2048, 64, seed=931)  # 64 work-groups only
    g = to_dev(d, dev)
    with pytest.raises(LiteLinearError) as ei:
        handle(dev).forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert ei.value.status == Status.UNSUPPORTED
