"""Pins of the oracle's GELU (tanh approximation), the activation that the
library's LITELINEAR_OPT_ACTIVATION fuses into the epilogue.

The definition (Hendrycks and Gimpel, "Gaussian Error Linear Units
(GELUs)", 2016, section 2) is pinned against what fixes it independently of
the oracle's formula:

* closed-form points and the identity gelu(v) - gelu(-v) = v, which holds
  for any function of the form v * (1 + odd(v)) / 2;
* the exact GELU v * Phi(v) (the approximation is within 5e-4 of it for
  every v);
* torch's own tanh-approximation GELU, an independent implementation, in
  float64;
* the tails (v for large v, 0 for large -v);
* the slope bound 1.13 that the GPU parity gate multiplies the forward's
  error by.

A plausible mistake in the oracle's formula (a dropped cubic term, a wrong
constant or sign, the sigmoid form with the wrong factor) fails one of them:
``test_pins_catch_planted_mistakes`` runs every pin on such variants.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

GRID = np.linspace(-12.0, 12.0, 48001)


def exact_gelu(v):
    return np.array([x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) for x in np.ravel(v)]).reshape(np.shape(v))


def pin_failures(f) -> list[str]:
    """Names of the pins that ``f`` fails."""
    bad = []
    if f(np.array([0.0]))[0] != 0.0:
        bad.append("zero")
    v = np.linspace(0.0, 8.0, 801)
    if np.max(np.abs((f(v) - f(-v)) - v)) > 1e-13:
        bad.append("odd identity")
    if np.max(np.abs(f(GRID) - exact_gelu(GRID))) > 5e-4:
        bad.append("exact GELU")
    t = torch.from_numpy(GRID)
    ref = torch.nn.functional.gelu(t, approximate="tanh").numpy()
    if np.max(np.abs(f(GRID) - ref) / np.maximum(np.abs(ref), 1e-300)) > 1e-12 and \
            np.max(np.abs(f(GRID) - ref)) > 1e-15:
        bad.append("torch tanh GELU")
    if abs(f(np.array([20.0]))[0] - 20.0) > 1e-12 or abs(f(np.array([-20.0]))[0]) > 1e-30:
        bad.append("tails")
    return bad


def test_oracle_gelu_meets_every_pin():
    assert pin_failures(oracle.gelu_tanh) == []


def test_hand_values():
    # 0.5 * 1 * (1 + tanh(sqrt(2/pi) * 1.044715)) worked by hand
    u = math.sqrt(2.0 / math.pi) * 1.044715
    assert abs(oracle.gelu_tanh(np.array([1.0]))[0] - 0.5 * (1.0 + math.tanh(u))) < 1e-16
    # gelu(-1) = gelu(1) - 1 (the odd identity at one point)
    assert abs(oracle.gelu_tanh(np.array([-1.0]))[0] - (0.5 * (1.0 + math.tanh(u)) - 1.0)) < 1e-16


def test_slope_bound_of_the_parity_gate():
    """|gelu(a) - gelu(b)| <= 1.13 |a - b|: the GPU gate for activated
    outputs scales the forward's error bound by 1.13."""
    g = oracle.gelu_tanh(GRID)
    slope = np.abs(np.diff(g) / np.diff(GRID))
    assert 1.12 < slope.max() <= 1.13


def test_pins_catch_planted_mistakes():
    c = math.sqrt(2.0 / math.pi)
    mutants = {
        "no cubic term": lambda v: 0.5 * v * (1.0 + np.tanh(c * v)),
        "cubic coefficient 0.04": lambda v: 0.5 * v * (1.0 + np.tanh(c * (v + 0.04 * v ** 3))),
        "sqrt(pi/2)": lambda v: 0.5 * v * (1.0 + np.tanh(math.sqrt(math.pi / 2) * (v + 0.044715 * v ** 3))),
        "minus inside": lambda v: 0.5 * v * (1.0 - np.tanh(c * (v + 0.044715 * v ** 3))),
        "sigmoid of u, not 2u": lambda v: v / (1.0 + np.exp(-c * (v + 0.044715 * v ** 3))),
        "exact erf GELU": exact_gelu,
        "float32 evaluation": lambda v: oracle.gelu_tanh(np.asarray(v, np.float32).astype(np.float64)
                                                         ).astype(np.float32).astype(np.float64),
    }
    for name, f in mutants.items():
        with np.errstate(over="ignore"):
            assert pin_failures(f), name
