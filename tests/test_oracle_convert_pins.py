"""Pins for the oracle's decomposition-side functions (the step upstream of the
forward: LiteLinear README, *Usage*, LiteLinear.from_dense; *Features*,
W ~ A.B + Q_fp8 with a per-tensor Q_scale_inv).

* The per-tensor quantiser against torch's own float8_e4m3fn cast (round to
  nearest even) of clamp(R / s, +-448) with s = amax / 448 in float32, on
  arrays built to hit ties, the subnormal range, signed zeros and the
  saturation edge.
* The residual W - A B against numpy's float64 matrix product.
* Planted mistakes must each fail at least one pin.
"""
from __future__ import annotations

import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
from oracle import build as oracle_build
from rank_fp8_residual_amd import workloads as wl


def _torch_quant(R: np.ndarray):
    Rt = torch.from_numpy(np.ascontiguousarray(R, dtype=np.float32))
    amax = float(Rt.abs().max()) if Rt.numel() else 0.0
    s = torch.tensor(amax, dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32) if amax > 0 else \
        torch.tensor(1.0, dtype=torch.float32)
    q = torch.clamp(Rt / s, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, float(s)


def quant_arrays():
    g = np.random.default_rng(3)
    arrs = [g.standard_normal(4096).astype(np.float32) * 0.02]
    # ties: with amax = 448 the scale is 1, and k/16 multiples of powers of two
    # sit halfway between e4m3fn neighbours
    ties = np.concatenate([np.arange(1, 64) * 2.0 ** e / 16 for e in range(-9, 9)]).astype(np.float32)
    arrs.append(np.concatenate([[448.0], ties, -ties, [0.0, -0.0]]).astype(np.float32))
    # wide dynamic range: most values fall into the subnormal codes or to zero
    arrs.append((g.standard_normal(4096) * np.exp2(g.integers(-40, 10, 4096))).astype(np.float32))
    arrs.append(np.zeros(64, np.float32))
    arrs.append(np.array([3.0e-38, -1.0e-30, 7.0], np.float32))
    # the ties again with amax = 448 2^e, so that the scale is exactly 2^e:
    # at the ends of and outside the range where a quantiser may divide by
    # way of a reciprocal (2^-60 .. 2^100), plus random values at those scales
    t = np.concatenate([np.arange(1, 64) * 2.0 ** e / 16 for e in range(-9, 5)])
    base = np.concatenate([[448.0], t, -t, g.standard_normal(2048) * 100.0])
    for e in (-90, -61, -60, 100, 101):
        arrs.append((base * 2.0 ** e).astype(np.float32))
    return arrs


def check_quant_vs_torch(lib):
    for R in quant_arrays():
        c, s = oracle.quantize_tensor(R, lib=lib)
        q, st = _torch_quant(R)
        assert s == st, (s, st)
        bad = np.nonzero(c != q)[0]
        assert bad.size == 0, (R[bad[:5]], c[bad[:5]], q[bad[:5]])


def check_quant_scale_and_range(lib):
    g = np.random.default_rng(4)
    R = (g.standard_normal(10000) * 0.05).astype(np.float32)
    c, s = oracle.quantize_tensor(R, lib=lib)
    assert s == np.float32(np.float32(np.abs(R).max()) / np.float32(448.0))
    dec = oracle.decode_e4m3fn(c, lib=lib) * s
    # every value within half an e4m3fn step of R (relative 2^-4, absolute 2^-10 s)
    assert np.all(np.abs(dec - R) <= np.maximum(np.abs(R) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6))
    assert np.max(np.abs(oracle.decode_e4m3fn(c, lib=lib))) == 448.0


def check_residual_vs_numpy(lib):
    d = wl.random_inputs(8, 96, 40, 12, seed=9)
    W = (torch.randn(40, 96, generator=torch.Generator().manual_seed(9)) * 0.1).to(torch.bfloat16)
    R = oracle.residual(W, d["A"], d["B"], lib=lib)
    ref = W.double().numpy() - d["A"].double().numpy() @ d["B"].double().numpy()
    assert np.allclose(R, ref, rtol=0, atol=1e-12)


CONVERT_PINS = [check_quant_vs_torch, check_quant_scale_and_range, check_residual_vs_numpy]


@pytest.mark.parametrize("pin", CONVERT_PINS, ids=lambda f: f.__name__)
def test_convert_pin(pin, oracle_lib):
    pin(oracle_lib)


CONVERT_PLANTS = {11: "B read transposed in the residual", 12: "scale from the e4m3fnuz maximum"}


@pytest.mark.parametrize("plant", sorted(CONVERT_PLANTS), ids=lambda p: CONVERT_PLANTS[p].replace(" ", "_"))
def test_convert_planted_mistake_is_caught(plant):
    with tempfile.TemporaryDirectory() as td:
        path = oracle_build.build(os.path.join(td, f"liboracle_plant{plant}.so"), plant=plant)
        lib = oracle.library(path)
        caught = []
        for pin in CONVERT_PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin catches planted mistake {plant}: {CONVERT_PLANTS[plant]}"
