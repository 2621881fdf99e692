"""GPU parity of the skinny path's all-of-K kernel (up to 16 rows, 2048 < in
<= 8192, at least 192 work-groups of 32 product columns): every work-group
streams its columns over all of K and T arrives in pieces from the lowest
work-groups.  Against the float64 oracle: ragged rows, column tails, K tails
(K not a multiple of the 1024-element wave quarter), ranks from none to 512,
the output and activation options and e4m3fnuz codes; repeat calls bit for
bit; the same inputs through the K-sliced kernels (a split-count hint turns
the all-of-K kernel off), which must also match the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Activation, Handle, Option, Path
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


def handle(dev, opts=None):
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(Path.SKINNY))
    for k, v in (opts or {}).items():
        h.set_option(k, v)
    return h


def fwd(h, g):
    y = h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    return y


def oracle_y(d, q_format="e4m3fn"):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"], d["scale"],
                          d["bias"], q_format=q_format)


FULLK_SHAPES = [  # M, in, out, r: 8 and 4 stages per wave, tails, rank counts
    (16, 8192, 8192, 64), (16, 8192, 8192, 0), (1, 8192, 8192, 64), (13, 4096, 8192, 200),
    (16, 6000, 8200, 64), (5, 2064, 7000, 16), (9, 8192, 6144, 512), (16, 3072, 6176, 80),
]


@pytest.mark.parametrize("shape", FULLK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_fullk_parity(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=1100 + M + r)
    say("fullk", shape, "f32" if out_f32 else "bf16")
    h = handle(dev, {Option.OUTPUT_F32: int(out_f32)})
    g = to_dev(d, dev)
    y1 = fwd(h, g)
    y2 = fwd(h, g)
    assert torch.equal(y1, y2)
    y_ref = oracle_y(d)
    parity.check(parity.to_f64(y1), y_ref, out_f32)
    # the K-sliced kernels on the same inputs
    say("fullk", shape, "K-sliced")
    hs = handle(dev, {Option.OUTPUT_F32: int(out_f32), Option.SPLIT_K: 4})
    parity.check(parity.to_f64(fwd(hs, g)), y_ref, out_f32)


def test_fullk_back_to_back_new_inputs(dev):
    """Two input sets of one shape queued back to back on one handle: the T
    pieces of the second launch are not those of the first."""
    M, K, N, r = 16, 8192, 8192, 64
    h = handle(dev)
    outs = []
    for seed in (1200, 1201, 1202):
        d = wl.random_inputs(M, K, N, r, seed=seed)
        g = to_dev(d, dev)
        say("fullk back to back", seed)
        outs.append((d, h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])))
    torch.cuda.synchronize()
    for d, y in outs:
        parity.check(parity.to_f64(y), oracle_y(d), False)


@pytest.mark.parametrize("variant", ["gelu", "geglu", "fnuz", "fnuz-geglu"])
def test_fullk_variants(dev, variant):
    fnuz = variant.startswith("fnuz")
    M, K, N, r = 11, 8192, 16384 if variant.endswith("geglu") else 8192, 64
    q_format = "e4m3fnuz" if fnuz else "e4m3fn"
    d = wl.random_inputs(M, K, N, r, seed=1300, q_format=q_format)
    opts = {Option.Q_FORMAT: int(fnuz)}
    if variant == "gelu":
        opts[Option.ACTIVATION] = int(Activation.GELU_TANH)
    if variant.endswith("geglu"):
        opts[Option.ACTIVATION] = int(Activation.GEGLU)
    say("fullk variant", variant)
    y = parity.to_f64(fwd(handle(dev, opts), to_dev(d, dev)))
    v_ref = oracle_y(d, q_format)
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
