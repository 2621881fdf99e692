"""GPU parity on seeded random shapes and option combinations, full output
against the float64 oracle: rows 1..700 (both paths, every tile size the
shapes select, ragged tails), in a multiple of 16 up to 3008, out up to
3000, ranks 0..130 (padded A for ranks that are not multiples of 8), and
ten shapes of the skinny path's all-of-K kernel, with
bf16 or float32 output, the GELU and gated epilogues, e4m3fnuz codes and the
fp8-activation mode drawn at random.  The draws are fixed by the seed, so the
cases are the same on every run; each case also repeats its call and must
agree bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Activation, Handle, Option
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


def draw_cases(n=40, seed=20261203):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 701))]))
        K = 16 * int(g.integers(1, 189))
        N = int(g.integers(1, 3001))
        r = int(g.choice([0, int(g.integers(1, 131)), 8 * int(g.integers(1, 9))]))
        act = str(g.choice(["none", "none", "gelu", "geglu"]))
        if act == "geglu":
            N += N % 2
        fnuz = bool(g.random() < 0.25)
        act8 = bool(not fnuz and g.random() < 0.2)
        cases.append(dict(i=i, M=M, K=K, N=N, r=r, act=act, fnuz=fnuz, act8=act8, f32=bool(g.random() < 0.3)))
    return cases


def draw_fullk_cases(n=10, seed=20261204, first=100):
    """Shapes of the skinny path's all-of-K kernel: up to 16 rows, 2048 < in
    <= 8192, at least 192 groups of 32 output columns (and the same option
    draws as above, without the fp8-activation mode, which runs tiled)."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(g.integers(1, 17))
        K = 16 * int(g.integers(129, 513))
        N = int(g.integers(6144, 10001))
        r = int(g.choice([0, int(g.integers(1, 131)), 16 * int(g.integers(1, 9))]))
        act = str(g.choice(["none", "none", "gelu", "geglu"]))
        if act == "geglu":
            N = 2 * N  # the gated epilogue's groups count output columns
        cases.append(dict(i=first + i, M=M, K=K, N=N, r=r, act=act, fnuz=bool(g.random() < 0.25), act8=False,
                          f32=bool(g.random() < 0.3)))
    return cases


CASES = draw_cases() + draw_fullk_cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['i']}-{c['M']}x{c['K']}x{c['N']}r{c['r']}")
def test_random_case(dev, case):
    M, K, N, r = case["M"], case["K"], case["N"], case["r"]
    q_format = "e4m3fnuz" if case["fnuz"] else "e4m3fn"
    d = wl.random_inputs(M, K, N, r, seed=5000 + case["i"], q_format=q_format)
    h = Handle(dev.index)
    h.set_option(Option.OUTPUT_F32, int(case["f32"]))
    h.set_option(Option.Q_FORMAT, int(case["fnuz"]))
    h.set_option(Option.ACT_FP8, int(case["act8"]))
    h.set_option(Option.ACTIVATION, {"none": 0, "gelu": int(Activation.GELU_TANH),
                                     "geglu": int(Activation.GEGLU)}[case["act"]])
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    say("random", case)
    args = (g["x"], g["A"] if r else None, g["B"] if r else None, g["Q"], g["scale"], g["bias"])
    y1 = h.forward(*args)
    y2 = h.forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y = parity.to_f64(y1)
    v_ref = oracle.forward(d["x"], d["A"] if r else None, d["B"] if r else None, d["Q"], d["scale"], d["bias"],
                           act_fp8=case["act8"], q_format=q_format)
    if case["act"] == "geglu":
        from tests.test_gpu_variants import check_geglu
        assert y.shape == (M, N // 2)
        check_geglu(y, v_ref, case["f32"])
    elif case["act"] == "gelu":
        y_ref = oracle.gelu_tanh(v_ref)
        rms = float(np.sqrt(np.mean(v_ref ** 2))) if v_ref.size else 0.0
        bound = 1.13 * parity.MAX_RMS_GATE * rms + (0.0 if case["f32"] else parity.half_ulp_bf16(y_ref))
        assert np.all(np.abs(y - y_ref) <= bound)
    else:
        parity.check(y, v_ref, case["f32"])
