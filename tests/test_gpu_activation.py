"""GPU parity of the fused activation (LITELINEAR_OPT_ACTIVATION = 1: GELU,
tanh approximation) against the oracle: gelu_tanh of the float64 forward.

Gate: the forward's gates (tests/parity.py) with the reference replaced by
gelu(y_ref) and the max bound's RMS taken from the pre-activation y_ref
times 1.13, the slope bound of the GELU pinned in
tests/test_oracle_activation_pins.py (an error d in y moves gelu(y) by at
most 1.13 d); the bf16 output's half-ulp is that of gelu(y_ref).  The
activation's own float32 evaluation (hardware exp2 and reciprocal, about
1 ulp each) is far inside it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Option, Path
from rank_fp8_residual_amd import workloads as wl
from tests import parity
from tests.test_gpu_parity import make_handle, run, sample_rows, say, to_dev
from tests.test_gpu_pair import make_pair, run_pair

pytestmark = pytest.mark.gpu

SLOPE = 1.13


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def check_gelu(y, y_pre, out_f32):
    rms = float(np.sqrt(np.mean(y_pre ** 2)))
    return parity.check(y, oracle.gelu_tanh(y_pre), out_f32, rms=SLOPE * rms)


def forward_ref(d, rows=None, act8=False):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"], d["scale"],
                          d["bias"], rows=rows, act_fp8=act8)


SHAPES = [  # M, in, out, r; path
    ((16, 2048, 1030, 64), Path.SKINNY), ((40, 512, 512, 32), Path.AUTO), ((64, 256, 256, 16), Path.AUTO),
    ((300, 1024, 520, 48), Path.TILED), ((513, 512, 700, 0), Path.TILED), ((1000, 768, 1030, 256), Path.TILED),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1].name)
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_gelu_parity(dev, case, out_f32):
    (M, K, N, r), path = case
    d = wl.random_inputs(M, K, N, r, seed=500 + M)
    say("gelu", (M, K, N, r), path.name, "f32" if out_f32 else "bf16")
    h = make_handle(dev, path, out_f32)
    h.set_option(Option.ACTIVATION, 1)
    y = parity.to_f64(run(h, to_dev(d, dev)))
    check_gelu(y, forward_ref(d), out_f32)
    # the same handle with the option off again gives the plain forward
    h.set_option(Option.ACTIVATION, 0)
    parity.check(parity.to_f64(run(h, to_dev(d, dev))), forward_ref(d), out_f32)


def test_gelu_256x256_tiles(dev):
    """The ping-pong loop's tiles (256 of 256 x 256) with the staged bf16
    epilogue; sampled rows."""
    M, K, N, r = 4096, 512, 4096, 64
    d = wl.random_inputs(M, K, N, r, seed=77)
    say("gelu 256x256", (M, K, N, r))
    h = make_handle(dev, Path.TILED)
    h.set_option(Option.ACTIVATION, 1)
    y = run(h, to_dev(d, dev))
    rows = sample_rows(M, 40)
    check_gelu(parity.to_f64(y[torch.from_numpy(rows).to(dev)]), forward_ref(d, rows=rows), False)


def test_gelu_with_e4m3fn_activations(dev):
    M, K, N, r = 512, 1024, 1024, 64
    d = wl.random_inputs(M, K, N, r, seed=78)
    say("gelu act8", (M, K, N, r))
    h = make_handle(dev, Path.TILED)
    h.set_option(Option.ACT_FP8, 1)
    h.set_option(Option.ACTIVATION, 1)
    y = parity.to_f64(run(h, to_dev(d, dev)))
    check_gelu(y, forward_ref(d, act8=True), False)


def test_gelu_pair(dev):
    d1, d2 = make_pair(700, 512, 520, 384, 48, seed=79)
    say("gelu pair")
    h = make_handle(dev, Path.TILED)
    h.set_option(Option.ACTIVATION, 1)
    y1, y2 = run_pair(h, d1, d2, dev)
    check_gelu(y1, forward_ref(d1), False)
    check_gelu(y2, forward_ref(d2), False)


@pytest.mark.parametrize("path", [Path.SKINNY, Path.TILED], ids=["skinny", "tiled"])
def test_gelu_of_bias_only(dev, path):
    """r = 0 and Q = 0: y = gelu(bias) exactly up to the activation's float32
    evaluation and the one rounding."""
    M, K, N = 32, 64, 300
    d = wl.random_inputs(M, K, N, 0, seed=80)
    d["Q"] = torch.zeros_like(d["Q"])
    d["bias"] = (torch.linspace(-6, 6, N, dtype=torch.float64)).to(torch.bfloat16)
    say("gelu bias only", path.name)
    h = make_handle(dev, path, out_f32=True)
    h.set_option(Option.ACTIVATION, 1)
    y = parity.to_f64(run(h, to_dev(d, dev)))
    expect = np.broadcast_to(oracle.gelu_tanh(d["bias"].to(torch.float64).numpy()), (M, N))
    # float32 evaluation: the exp2 argument 2 u log2(e) reaches 36 at -6, so
    # its rounding alone moves the tail's relative value by up to ~4e-6
    assert np.max(np.abs(y - expect) / np.maximum(np.abs(expect), 1e-30)) < 1e-5
