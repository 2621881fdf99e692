"""Pins of the oracle's e4m3fnuz decode and of its forward on e4m3fnuz codes.

The LiteLinear README (Features) names e4m3fnuz as the residual's format on
AMD hardware, beside e4m3fn on NVIDIA.  The oracle's closed form is checked
against what fixes the format independently of it:

* torch's own float8_e4m3fnuz conversion on all 256 codes;
* closed-form points of the format: bias 8, largest value 240 at 0x7F (and
  -240 at 0xFF), subnormals f * 2^-10, 0x80 the only NaN, no negative zero;
* the relation to the (separately pinned) e4m3fn decode: every code but
  0x7F, 0xFF and 0x80 decodes to exactly half its e4m3fn value;
* the forward on e4m3fnuz codes against numpy float64 with torch's decode.

A planted mistake (the e4m3fn exponent bias) must fail them.
"""
from __future__ import annotations

import math
import os
import tempfile

import numpy as np
import torch

import oracle
from oracle import build as oracle_build
from rank_fp8_residual_amd import workloads as wl


def torch_fnuz(codes) -> np.ndarray:
    c = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return c.view(torch.float8_e4m3fnuz).to(torch.float64).numpy()


def pin_all_codes_vs_torch(lib):
    mine = oracle.decode_e4m3fnuz(np.arange(256), lib=lib)
    ref = torch_fnuz(np.arange(256))
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def pin_closed_form_points(lib):
    dec = lambda c: lib.oracle_e4m3fnuz_to_f64(c)
    assert dec(0x7F) == 240.0 and dec(0xFF) == -240.0
    assert dec(0x01) == 2.0 ** -10 and dec(0x81) == -(2.0 ** -10)
    assert dec(0x07) == 7 * 2.0 ** -10 and dec(0x08) == 2.0 ** -7
    assert dec(0x40) == 1.0 and dec(0x38) == 0.5 and dec(0x47) == 1.875
    assert dec(0x00) == 0.0 and not math.copysign(1.0, dec(0x00)) < 0
    assert math.isnan(dec(0x80))
    assert sum(math.isnan(dec(c)) for c in range(256)) == 1
    vals = [dec(c) for c in range(0x00, 0x80)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # monotone over the positive codes


def pin_half_of_e4m3fn(lib):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)])
    assert np.array_equal(oracle.decode_e4m3fnuz(codes, lib=lib), 0.5 * oracle.decode_e4m3fn(codes, lib=lib))


def pin_forward_vs_numpy(lib):
    d = wl.random_inputs(9, 96, 40, 8, seed=31)
    # every code, including +-240 and subnormals (0x80, the NaN, left out)
    g = np.random.Generator(np.random.PCG64(32))
    codes = g.choice(np.array([c for c in range(256) if c != 0x80], np.uint8), size=(40, 96))
    codes[0, :4] = [0x7F, 0xFF, 0x01, 0x81]
    Q = torch.from_numpy(codes)
    y = oracle.forward(d["x"], d["A"], d["B"], Q, d["scale"], d["bias"], q_format="e4m3fnuz", lib=lib)
    x = d["x"].to(torch.float64).numpy()
    A, B = d["A"].to(torch.float64).numpy(), d["B"].to(torch.float64).numpy()
    ref = (x @ B.T) @ A.T + float(np.float32(d["scale"])) * (x @ torch_fnuz(codes).T) + d["bias"].double().numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # and differs from reading the same bytes as e4m3fn
    y_fn = oracle.forward(d["x"], d["A"], d["B"], Q, d["scale"], d["bias"], lib=lib)
    assert not np.allclose(y, y_fn)


PINS = [pin_all_codes_vs_torch, pin_closed_form_points, pin_half_of_e4m3fn, pin_forward_vs_numpy]


def test_pins(oracle_lib):
    for pin in PINS:
        pin(oracle_lib)


def test_nan_code_propagates(oracle_lib):
    d = wl.random_inputs(3, 32, 5, 0, seed=33)
    Q = torch.zeros((5, 32), dtype=torch.uint8)
    Q[2, 7] = 0x80
    y = oracle.forward(d["x"], None, None, Q, d["scale"], d["bias"], q_format="e4m3fnuz", lib=oracle_lib)
    assert np.all(np.isnan(y[:, 2])) and np.all(np.isfinite(np.delete(y, 2, axis=1)))


def test_planted_fn_bias_is_caught():
    with tempfile.TemporaryDirectory() as td:
        lib = oracle.library(oracle_build.build(os.path.join(td, "liboracle_plant13.so"), plant=13))
        caught = []
        for pin in PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught
