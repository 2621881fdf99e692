"""GPU parity of litelinear_forward_pair (two outputs sharing x and B, T
computed once) against two float64 oracle forwards, with the gates of
tests/parity.py.  Covers different widths and scales per output, a missing
bias, r = 0, wide T blocks, an unfoldable scale (the 128 x 128 order), the
skinny regime (one forward per output), exact inputs (bit for bit), the
float32 output, e4m3fn activations, and one handle alternating single and
pair calls.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Handle, LiteLinearError, Option, Status
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


def make_pair(M, K, N1, N2, r, seed, exact=False, with_bias2=True):
    mk = wl.exact_inputs if exact else wl.random_inputs
    d1 = mk(M, K, N1, r, seed=seed)
    d2 = mk(M, K, N2, r, seed=seed + 1)
    d2["x"], d2["B"] = d1["x"], d1["B"]  # shared
    if not with_bias2:
        d2["bias"] = None
    if not exact:
        d2["scale"] = d1["scale"] * 1.75
    return d1, d2


def oracle_y(d, act8=False):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"], d["scale"],
                          d["bias"], act_fp8=act8)


def run_pair(h, d1, d2, dev):
    t = lambda v: v.to(dev) if isinstance(v, torch.Tensor) else v
    r = d1["r"]
    y1, y2 = h.forward_pair(t(d1["x"]), t(d1["B"]) if r else None,
                            (t(d1["A"]) if r else None, t(d1["Q"]), d1["scale"], t(d1["bias"])),
                            (t(d2["A"]) if r else None, t(d2["Q"]), d2["scale"], t(d2["bias"])))
    torch.cuda.synchronize()
    return parity.to_f64(y1), parity.to_f64(y2)


PAIR_SHAPES = [  # M, in, out1, out2, r
    (300, 512, 520, 384, 48), (1000, 768, 1030, 1030, 64), (513, 1024, 256, 700, 256), (700, 256, 300, 200, 0),
    (2048, 1024, 2048, 4096, 64),
]


@pytest.mark.parametrize("shape", PAIR_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_pair_parity(dev, shape, out_f32):
    M, K, N1, N2, r = shape
    d1, d2 = make_pair(M, K, N1, N2, r, seed=300 + M, with_bias2=(M % 2 == 0))
    say("pair", shape, "f32" if out_f32 else "bf16")
    h = Handle(dev.index)
    h.set_option(Option.OUTPUT_F32, int(out_f32))
    y1, y2 = run_pair(h, d1, d2, dev)
    parity.check(y1, oracle_y(d1), out_f32)
    parity.check(y2, oracle_y(d2), out_f32)


def test_pair_unfoldable_scale(dev):
    d1, d2 = make_pair(300, 256, 256, 320, 32, seed=11)
    d2["scale"] = 2.0 ** -70  # outside the folding range: both outputs take the unfolded order
    say("pair unfoldable scale")
    y1, y2 = run_pair(Handle(dev.index), d1, d2, dev)
    parity.check(y1, oracle_y(d1), False)
    parity.check(y2, oracle_y(d2), False)


def test_pair_skinny_regime(dev):
    d1, d2 = make_pair(16, 2048, 640, 512, 64, seed=12)
    say("pair skinny")
    y1, y2 = run_pair(Handle(dev.index), d1, d2, dev)
    parity.check(y1, oracle_y(d1), False)
    parity.check(y2, oracle_y(d2), False)


@pytest.mark.parametrize("shape", [(300, 512, 260, 384, 64), (257, 256, 513, 64, 16)],
                         ids=lambda s: "x".join(map(str, s)))
def test_pair_exact_bitwise(dev, shape):
    M, K, N1, N2, r = shape
    d1, d2 = make_pair(M, K, N1, N2, r, seed=13, exact=True)
    say("pair exact", shape)
    h = Handle(dev.index)
    h.set_option(Option.OUTPUT_F32, 1)
    y1, y2 = run_pair(h, d1, d2, dev)
    assert np.array_equal(y1, oracle_y(d1)) and np.array_equal(y2, oracle_y(d2))


def test_pair_act_fp8(dev):
    d1, d2 = make_pair(600, 1024, 768, 512, 64, seed=14)
    say("pair act8")
    h = Handle(dev.index)
    h.set_option(Option.ACT_FP8, 1)
    y1, y2 = run_pair(h, d1, d2, dev)
    parity.check(y1, oracle_y(d1, act8=True), False)
    parity.check(y2, oracle_y(d2, act8=True), False)


def test_pair_and_single_calls_share_a_handle(dev):
    """Single and pair calls alternate on one handle (the T-ready counters
    keep one layout per shape; the pair adds its second T' workspace)."""
    d1, d2 = make_pair(300, 512, 520, 384, 64, seed=15)
    ref1, ref2 = oracle_y(d1), oracle_y(d2)
    h = Handle(dev.index)
    t = lambda v: v.to(dev) if isinstance(v, torch.Tensor) else v
    for rep in range(3):
        say("pair/single alternation", rep)
        y = h.forward(t(d1["x"]), t(d1["A"]), t(d1["B"]), t(d1["Q"]), d1["scale"], t(d1["bias"]))
        torch.cuda.synchronize()
        parity.check(parity.to_f64(y), ref1, False)
        y1, y2 = run_pair(h, d1, d2, dev)
        parity.check(y1, ref1, False)
        parity.check(y2, ref2, False)


def test_pair_rejects_overlapping_outputs(dev):
    d1, d2 = make_pair(64, 256, 128, 128, 16, seed=16)
    t = lambda v: v.to(dev) if isinstance(v, torch.Tensor) else v
    h = Handle(dev.index)
    y = torch.empty((64, 128), dtype=torch.bfloat16, device=dev)
    say("pair overlap")
    with pytest.raises(LiteLinearError) as e:
        h.forward_pair(t(d1["x"]), t(d1["B"]), (t(d1["A"]), t(d1["Q"]), d1["scale"], t(d1["bias"])),
                       (t(d2["A"]), t(d2["Q"]), d2["scale"], t(d2["bias"])), out=(y, y))
    assert e.value.status == Status.INVALID_ARG
