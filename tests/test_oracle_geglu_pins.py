"""Pins of the oracle's exact GELU and GEGLU, the gated activation that the
library's LITELINEAR_OPT_ACTIVATION = 2 fuses into the epilogue.

GELU(v) = v Phi(v) (Hendrycks and Gimpel, 2016, section 2) and
GEGLU(y) = hidden * GELU(gate) over the two halves of a projection's output
(Shazeer, "GLU Variants Improve Transformer", 2020; the LiteLinear README's
integration guide passes such an activation projection through LiteLinear).
They are pinned against:

* closed-form points: GELU(0) = 0, GELU(1) = Phi(1), GELU(v) - GELU(-v) = v;
* torch's own exact GELU (approximate='none') in float64, an independent
  implementation, over [-12, 12];
* the tails (v for large v, 0 for large -v);
* the slope bound used by the GPU gate (the exact GELU's largest slope is
  about 1.129);
* GEGLU against torch on both halves computed independently (hidden from the
  first F columns, the gate from the last F), on a hand-checkable case too.

Planted mistakes (the tanh approximation in place of erf, erf(v) without the
1/sqrt(2), the halves swapped, the gate not gated) each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

GRID = np.linspace(-12.0, 12.0, 24001)


def gelu_failures(f) -> list[str]:
    bad = []
    try:
        assert f(np.array([0.0]))[0] == 0.0
        phi1 = 0.5 * (1.0 + math.erf(1.0 / math.sqrt(2.0)))
        assert abs(f(np.array([1.0]))[0] - phi1) < 1e-15
    except AssertionError:
        bad.append("points")
    v = np.linspace(0.0, 8.0, 801)
    if not np.allclose(f(v) - f(-v), v, rtol=0, atol=1e-14):
        bad.append("odd part")
    ref = torch.nn.functional.gelu(torch.from_numpy(GRID), approximate="none").numpy()
    if not np.allclose(f(GRID), ref, rtol=1e-13, atol=1e-15):
        bad.append("torch")
    if not (f(np.array([30.0]))[0] == 30.0 and abs(f(np.array([-30.0]))[0]) < 1e-150):
        bad.append("tails")
    slope = np.max(np.diff(f(GRID)) / np.diff(GRID))
    if not 1.12 < slope <= 1.13:
        bad.append("slope")
    return bad


def test_gelu_erf_pins():
    assert gelu_failures(oracle.gelu_erf) == []


def test_gelu_pins_catch_planted_mistakes():
    from scipy.special import erf
    plants = {
        "tanh approximation": oracle.gelu_tanh,
        "erf without 1/sqrt(2)": lambda v: 0.5 * v * (1.0 + erf(v)),
        "float32": lambda v: oracle.gelu_erf(np.asarray(v, np.float32).astype(np.float32)).astype(np.float32)
        .astype(np.float64),
        "sigmoid form": lambda v: v / (1.0 + np.exp(-1.702 * v)),
    }
    for name, f in plants.items():
        assert gelu_failures(f), name


def geglu_failures(g) -> list[str]:
    bad = []
    # hand-checkable: hidden 2, gate 1 -> 2 Phi(1); hidden -3, gate 0 -> 0
    y = np.array([[2.0, -3.0, 1.0, 0.0]])
    phi1 = 0.5 * (1.0 + math.erf(1.0 / math.sqrt(2.0)))
    out = g(y)
    if out.shape != (1, 2) or abs(out[0, 0] - 2.0 * phi1) > 1e-15 or out[0, 1] != 0.0:
        bad.append("hand")
    rng = np.random.Generator(np.random.PCG64(5))
    y = rng.standard_normal((7, 2 * 13)) * 3.0
    h, gate = torch.from_numpy(y[:, :13].copy()), torch.from_numpy(y[:, 13:].copy())
    ref = (h * torch.nn.functional.gelu(gate, approximate="none")).numpy()
    o = g(y)
    if o.shape != ref.shape or not np.allclose(o, ref, rtol=1e-13, atol=1e-15):
        bad.append("torch")
    return bad


def test_geglu_pins():
    assert geglu_failures(oracle.geglu) == []


def test_geglu_pins_catch_planted_mistakes():
    F = lambda y: np.asarray(y).shape[-1] // 2
    plants = {
        "halves swapped": lambda y: y[..., F(y):] * oracle.gelu_erf(y[..., :F(y)]),
        "not gated": lambda y: oracle.gelu_erf(y[..., F(y):]),
        "gelu on both": lambda y: oracle.gelu_erf(y[..., :F(y)]) * oracle.gelu_erf(y[..., F(y):]),
        "interleaved halves": lambda y: y[..., 0::2] * oracle.gelu_erf(y[..., 1::2]),
    }
    for name, g in plants.items():
        assert geglu_failures(g), name
