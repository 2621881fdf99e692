"""GPU parity of the fp8-activation mode (LITELINEAR_OPT_ACT_FP8) and of
litelinear_quantize_rows, through the C ABI, against the float64 oracle.

* The quantiser is integer work: codes and scales must equal the oracle's
  bit for bit (all finite bf16 values up to 448, rows across the whole
  exponent range, subnormal rows, signed zeros, all-zero and non-finite rows).
* The forward is checked against the oracle's fp8-activation forward with the
  same gates as the bf16 forward (tests/parity.py): both take the same
  quantisation decisions, and every fp8 product is exact.
* Inputs whose activations quantise exactly must agree bit for bit.
* The method's own error (fp8 activations against the exact bf16-activation
  forward) stays inside its stated tolerance: max <= 0.25 RMS(y) (+ half a
  bf16 ulp) and relative L1 <= 4e-2.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Handle, Kernel, LiteLinearError, Option, Path, Status
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


def to_dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def act8_handle(dev, out_f32=False):
    h = Handle(dev.index)
    h.set_option(Option.ACT_FP8, 1)
    h.set_option(Option.OUTPUT_F32, int(out_f32))
    return h


def run(h, g):
    y = h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    return y


def oracle_y8(d, rows=None):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"],
                          d["scale"], d["bias"], rows=rows, act_fp8=True)


def quant_cases():
    """Row sets for the quantiser: (name, bf16 [M, K])."""
    cases = []
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = bits.to(torch.float64)
    vals = bits[torch.isfinite(v) & (v.abs() <= 448)]
    width = 128
    rows = (vals.numel() + width - 2) // (width - 1)
    x = torch.zeros(rows, width, dtype=torch.bfloat16)
    x[:, 0] = 448.0
    flat = torch.zeros(rows * (width - 1), dtype=torch.bfloat16)
    flat[:vals.numel()] = vals
    x[:, 1:] = flat.view(rows, width - 1)
    cases.append(("all bf16 up to 448", x))
    g = torch.Generator().manual_seed(21)
    M, K = 301, 1024
    sig = torch.pow(2.0, torch.randint(-140, 121, (M, 1), generator=g).to(torch.float64))
    xr = torch.randn(M, K, generator=g, dtype=torch.float64) * sig
    xr[5] = 0.0
    xr[6] = -0.0
    xr[7, ::3] = -0.0
    xr[8] = torch.randn(K, generator=g, dtype=torch.float64) * 2.0 ** -133   # bf16 subnormals
    xr[9, 17] = 448.0 * 2.0 ** 3                                           # on a scale boundary
    xr[10, 3] = 448.0 * 2.0 ** 3 * (1 + 2 ** -7)                            # just above it
    xr[11, :] = 1.0
    xr[11, 40] = float("nan")
    xr[12, 0] = float("inf")
    xr[13, 100] = -float("inf")
    xr[14, :10] = 3.0e38
    cases.append(("random magnitudes", xr.to(torch.bfloat16)))
    cases.append(("short rows", (torch.randn(7, 16, generator=g) * 50).to(torch.bfloat16)))
    cases.append(("long rows", torch.randn(5, 8192, generator=g).to(torch.bfloat16)))
    return cases


@pytest.mark.parametrize("case", range(4))
def test_quantize_rows_bit_exact(dev, case):
    name, x = quant_cases()[case]
    say("quantize_rows", name, tuple(x.shape))
    codes, scales = Handle(dev.index).quantize_rows(x.to(dev))
    torch.cuda.synchronize()
    c_ref, e_ref = oracle.quantize_rows(x)
    c = codes.cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, (name, bad[:5].tolist(), c[tuple(bad[0])], c_ref[tuple(bad[0])],
                           float(x[tuple(bad[0])]))
    s_ref = np.ldexp(np.float32(1.0), e_ref.astype(np.int64)).astype(np.float32)
    s_ref[np.all(c_ref == 0x7F, axis=1) & (e_ref == 0)] = 1.0
    assert np.array_equal(scales.cpu().numpy(), s_ref), name


ACT8_SHAPES = [  # M, in, out, r: several tiles, ragged tails, K not a multiple of 128
    (1, 256, 300, 16), (37, 1040, 777, 64), (300, 2048, 520, 48), (513, 512, 700, 64),
    (1000, 768, 1030, 256), (260, 4096, 256, 0),
]


@pytest.mark.parametrize("shape", ACT8_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_act8_random_parity(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=2000 + M)
    y_ref = oracle_y8(d)
    say("act8 random", shape, "f32" if out_f32 else "bf16")
    y = parity.to_f64(run(act8_handle(dev, out_f32), to_dev(d, dev)))
    parity.check(y, y_ref, out_f32)


@pytest.mark.parametrize("shape", [(16, 64, 256, 16), (257, 512, 513, 64), (300, 2048, 64, 128),
                                   (4096, 256, 4096, 64), (3630, 256, 8192, 512), (2048, 256, 4096, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_act8_exact_inputs_bitwise(dev, shape):
    """Integer activations in [-4, 4] quantise exactly (scale 2^-6), so the
    fp8-activation forward is the exact forward, bit for bit."""
    M, K, N, r = shape
    d = wl.exact_inputs(M, K, N, r, seed=M + K)
    y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"])
    assert np.array_equal(oracle_y8(d), y_ref)
    g = to_dev(d, dev)
    for out_f32 in (True, False):
        say("act8 exact", shape, out_f32)
        y = parity.to_f64(run(act8_handle(dev, out_f32), g))
        expect = y_ref if out_f32 else parity.bf16_of(y_ref)
        bad = np.argwhere(y != expect)
        assert bad.size == 0, (bad[:5].tolist(), y[tuple(bad[0])], expect[tuple(bad[0])])


# Full-size workloads in this mode are compared over their whole outputs in
# tests/test_gpu_full.py.


def test_act8_nonfinite_rows(dev):
    d = wl.random_inputs(40, 512, 300, 16, seed=31)
    d["x"][3, 7] = float("nan")
    d["x"][20, 0] = float("inf")
    say("act8 non-finite rows")
    y = run(act8_handle(dev), to_dev(d, dev)).cpu().to(torch.float64)
    assert bool(torch.isnan(y[3]).all()) and bool(torch.isnan(y[20]).all())
    keep = [i for i in range(40) if i not in (3, 20)]
    y_ref = oracle_y8(d, rows=keep)
    parity.check(y[keep].numpy(), y_ref, False)


def test_act8_handle_switches_modes(dev):
    """One handle alternating between bf16 and fp8 activations (and shapes)."""
    h = Handle(dev.index)
    cases = [wl.random_inputs(300, 512, 512, 64, seed=41), wl.random_inputs(700, 256, 384, 32, seed=42)]
    for rep in range(2):
        for i, d in enumerate(cases):
            for act8 in (0, 1):
                say("act8 switch", rep, i, act8)
                h.set_option(Option.ACT_FP8, act8)
                y = parity.to_f64(run(h, to_dev(d, dev)))
                ref = oracle_y8(d) if act8 else oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"],
                                                               d["bias"])
                parity.check(y, ref, False)


def test_act8_options_and_errors(dev):
    say("act8 options")
    h = Handle(dev.index)
    for bad in (2, -1):
        with pytest.raises(LiteLinearError) as e:
            h.set_option(Option.ACT_FP8, bad)
        assert e.value.status == Status.INVALID_ARG
    d = to_dev(wl.random_inputs(16, 256, 64, 8, seed=43), dev)
    h.set_option(Option.ACT_FP8, 1)
    h.set_option(Option.PATH, int(Path.SKINNY))
    with pytest.raises(LiteLinearError) as e:
        h.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"])
    assert e.value.status == Status.UNSUPPORTED
    h.set_option(Option.PATH, int(Path.AUTO))
    h.set_option(Option.PROFILE, 1)
    run(h, d)
    assert h.kernel_time(Kernel.QUANT)[1] == 1 and h.kernel_time(Kernel.MAIN)[1] == 1
    with pytest.raises(LiteLinearError) as e:  # codes must not overlap x
        h.quantize_rows(d["x"], codes=d["x"].view(torch.uint8).view(-1)[:16 * 256].view(16, 256))
    assert e.value.status == Status.INVALID_ARG
    with pytest.raises(LiteLinearError) as e:  # in % 16 != 0
        h.quantize_rows(torch.zeros((4, 24), dtype=torch.bfloat16, device=dev))
    assert e.value.status == Status.UNSUPPORTED
