"""Pins for the oracle's fp8-activation mode (activations quantised to e4m3fn
with one power-of-two scale per row before the residual product).

* The quantiser against brute force: every finite bf16 value of magnitude at
  most 448, in rows whose scale is 2^0, must map to the e4m3fn value nearest
  to it (all 127 magnitudes tried; ties to the even code), with its sign.
  The e4m3fn values come from torch's float8_e4m3fn conversion, not from the
  oracle.
* The scale exponent is the smallest one that keeps the row inside +-448,
  checked at and around the powers-of-two boundaries.
* Activations that are already 2^k times e4m3fn values quantise exactly, so
  the mode's forward equals the plain forward there.
* The mode's forward equals a numpy evaluation of its definition: T from the
  bf16 x, the residual product from the quantised x.
* Planted mistakes in the oracle's source must each fail at least one pin.
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


def _e4m3_magnitudes() -> np.ndarray:
    """The 127 finite non-negative e4m3fn values, indexed by code 0x00..0x7E."""
    return torch.arange(0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _brute_nearest(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each |v| <= 448 by exhaustive search, ties to
    the even code, sign bit from v."""
    mags = _e4m3_magnitudes()
    a = np.abs(v)[:, None]
    dist = np.abs(a - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates the even code wins (at most two candidates tie)
    even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def _all_bf16_up_to_448() -> torch.Tensor:
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = bits.to(torch.float64)
    keep = torch.isfinite(v) & (v.abs() <= 448)
    return bits[keep]


def check_quant_nearest_all_bf16(lib):
    vals = _all_bf16_up_to_448()
    n = vals.numel()
    width = 64
    rows = (n + width - 2) // (width - 1)
    # every row starts with 448, so its scale is 2^0 and codes are nearest values
    x = torch.zeros(rows, width, dtype=torch.bfloat16)
    x[:, 0] = 448.0
    flat = torch.zeros(rows * (width - 1), dtype=torch.bfloat16)
    flat[:n] = vals
    x[:, 1:] = flat.view(rows, width - 1)
    codes, exps = oracle.quantize_rows(x, lib=lib)
    assert np.all(exps == 0), np.unique(exps)
    got = codes[:, 1:].reshape(-1)[:n]
    want = _brute_nearest(vals.to(torch.float64).numpy())
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (vals[bad[:5]].tolist(), got[bad[:5]], want[bad[:5]])


def check_scale_exponent_minimal(lib):
    base = [448.0 * 2.0 ** k for k in (-130, -20, -7, -1, 0, 1, 5, 100)]
    amaxes = []
    for b in base:
        for f in (1.0, 1.0 + 2 ** -7, 1.0 - 2 ** -8, 0.5, 0.875 / 0.875 * 1.5, 1.75):
            amaxes.append(b * f)
    amaxes += [0.0, 1e-40, 3.0e38, 1.0, 2.0 ** -126]
    x = torch.zeros(len(amaxes), 16, dtype=torch.float64)
    x[:, 3] = torch.tensor(amaxes, dtype=torch.float64)
    x[:, 7] = -torch.tensor(amaxes, dtype=torch.float64) / 3
    xb = x.to(torch.bfloat16)
    codes, exps = oracle.quantize_rows(xb, lib=lib)
    amax = xb.to(torch.float64).abs().max(dim=1).values.numpy()
    for a, e in zip(amax, exps):
        assert e >= -126
        assert a <= 448.0 * 2.0 ** int(e), (a, e)
        if a > 0 and e > -126:
            assert a > 448.0 * 2.0 ** (int(e) - 1), (a, e)
        if a == 0:
            assert e == -126
    # and the codes stay finite (no code beyond 448)
    assert not np.any((codes & 0x7F) == 0x7F)


def check_exact_inputs_match_plain_forward(lib):
    g = torch.Generator().manual_seed(5)
    M, K, N, r = 6, 64, 24, 8
    codes = torch.randint(0, 0x7F, (M, K), generator=g, dtype=torch.int32)
    codes[:, 0] = 0x7E  # 448: the row's scale is exactly 2^k
    sign = torch.randint(0, 2, (M, K), generator=g, dtype=torch.int32) << 7
    vals = (codes | sign).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    ks = torch.tensor([-9, -3, 0, 2, 7, 20], dtype=torch.float64)[:, None]
    x = (vals * 2.0 ** ks).to(torch.bfloat16)
    assert torch.equal(x.to(torch.float64), vals * 2.0 ** ks)  # exact in bf16
    d = wl.random_inputs(M, K, N, r, seed=6)
    y8 = oracle.forward(x, d["A"], d["B"], d["Q"], d["scale"], d["bias"], act_fp8=True, lib=lib)
    y = oracle.forward(x, d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
    assert np.array_equal(y8, y)
    c, e = oracle.quantize_rows(x, lib=lib)
    assert np.array_equal(e, ks[:, 0].numpy().astype(np.int32))


def check_definition_vs_numpy(lib):
    d = wl.random_inputs(9, 96, 40, 12, seed=7)
    y8, T8 = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], act_fp8=True,
                            want_T=True, lib=lib)
    codes, exps = oracle.quantize_rows(d["x"], lib=lib)
    xq = oracle.decode_e4m3fn(codes, lib=lib) * np.ldexp(1.0, exps.astype(np.int64))[:, None]
    x = d["x"].to(torch.float64).numpy()
    A = d["A"].to(torch.float64).numpy()
    B = d["B"].to(torch.float64).numpy()
    Qv = d["Q"].view(torch.float8_e4m3fn).to(torch.float64).numpy()
    bias = d["bias"].to(torch.float64).numpy()
    T = x @ B.T
    y = T @ A.T + float(d["scale"]) * (xq @ Qv.T) + bias
    assert np.allclose(T8, T, rtol=1e-12, atol=1e-12)
    assert np.allclose(y8, y, rtol=1e-10, atol=1e-10), np.abs(y8 - y).max()
    # the quantised activations are close to x: within one e4m3fn step
    step = np.ldexp(1.0, exps.astype(np.int64))[:, None] * 2.0 ** -3 * np.maximum(
        np.abs(xq) / np.ldexp(1.0, exps.astype(np.int64))[:, None], 2.0 ** -6)
    assert np.all(np.abs(xq - x) <= step + 1e-300)


def check_nonfinite_row(lib):
    d = wl.random_inputs(4, 32, 8, 4, seed=8)
    x = d["x"].clone()
    x[1, 5] = float("nan")
    x[2, 0] = float("inf")
    codes, exps = oracle.quantize_rows(x, lib=lib)
    assert np.all(codes[1] == 0x7F) and np.all(codes[2] == 0x7F) and exps[1] == 0 and exps[2] == 0
    assert not np.any(codes[0] == 0x7F) and not np.any(codes[3] == 0x7F)
    y = oracle.forward(x, d["A"], d["B"], d["Q"], d["scale"], d["bias"], act_fp8=True, lib=lib)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    assert np.all(np.isfinite(y[0])) and np.all(np.isfinite(y[3]))


ACT8_PINS = [check_quant_nearest_all_bf16, check_scale_exponent_minimal, check_exact_inputs_match_plain_forward,
             check_definition_vs_numpy, check_nonfinite_row]


@pytest.mark.parametrize("pin", ACT8_PINS, ids=lambda f: f.__name__)
def test_act8_pin(pin, oracle_lib):
    pin(oracle_lib)


ACT8_PLANTS = {8: "ties away from zero", 9: "scale leaves amax above 448", 10: "T from the quantised x"}


@pytest.mark.parametrize("plant", sorted(ACT8_PLANTS), ids=lambda p: ACT8_PLANTS[p].replace(" ", "_"))
def test_act8_planted_mistake_is_caught(plant):
    with tempfile.TemporaryDirectory() as td:
        path = oracle_build.build(os.path.join(td, f"liboracle_plant{plant}.so"), plant=plant)
        lib = oracle.library(path)
        caught = []
        for pin in ACT8_PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin catches planted mistake {plant}: {ACT8_PLANTS[plant]}"
