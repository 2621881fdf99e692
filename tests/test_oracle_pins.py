"""Pins for the CPU oracle: it is checked against things fixed by the format,
by the mathematics and by independent library routines, never against itself.

* e4m3fn decode: torch's own float8_e4m3fn conversion on all 256 codes, and
  closed-form points of the OCP format (LiteLinear README, Features: the
  residual is e4m3fn).
* Q = 0 reduces the forward to the textbook two-matmul low-rank layer
  (tt_compressor page, SVDLinearLayer: y = (x @ B.T) @ A.T + bias).
* A = B = 0, and r = 0, reduce it to a scaled matmul with the decoded residual.
* The dense product x (A B + scale dec(Q))^T + bias equals it by associativity
  (README introduction: W ~ A.B + scale.Q).
* Exact rational brute force on tiny inputs, exact integer inputs, and
  invariants (linearity, bias shift, scale doubling, row permutation).
* Planted mistakes in the oracle's source must each fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import build as oracle_build
from rank_fp8_residual_amd import workloads as wl


def _f64(t):
    return t.detach().to(torch.float64).numpy()


def _torch_dec(Q: torch.Tensor) -> np.ndarray:
    return Q.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- decode pins

def check_decode_vs_torch(lib):
    codes = np.arange(256)
    mine = oracle.decode_e4m3fn(codes, lib=lib)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_m, nan_r = np.isnan(mine), np.isnan(ref)
    assert np.array_equal(nan_m, nan_r), np.nonzero(nan_m != nan_r)
    assert np.array_equal(mine[~nan_m], ref[~nan_r])
    assert np.array_equal(np.signbit(mine[~nan_m]), np.signbit(ref[~nan_r]))


def test_decode_matches_torch_all_codes(oracle_lib):
    check_decode_vs_torch(oracle_lib)


def test_decode_closed_form_points(oracle_lib):
    d = lambda c: oracle.decode_e4m3fn([c], lib=oracle_lib)[0]
    assert d(0x00) == 0.0 and not math.copysign(1, d(0x00)) < 0
    assert d(0x80) == 0.0 and math.copysign(1, d(0x80)) < 0
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x3C) == 1.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))


def test_decode_monotone_and_bf16_exact(oracle_lib):
    pos = oracle.decode_e4m3fn(np.arange(0, 0x7F), lib=oracle_lib)
    assert np.all(np.diff(pos) > 0)
    neg = oracle.decode_e4m3fn(np.arange(0x80, 0xFF), lib=oracle_lib)
    assert np.array_equal(neg, -pos)
    finite = np.concatenate([pos, neg])
    rt = torch.from_numpy(finite).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rt, finite)  # every e4m3fn value is exact in bf16


def test_bf16_decode_all_patterns(oracle_lib):
    lib = oracle_lib
    bits = torch.arange(0, 65536, 97, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([lib.oracle_bf16_to_f64(int(b) & 0xFFFF) for b in bits.numpy()])
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.array_equal(mine[~both_nan], ref[~both_nan])


# --------------------------------------------------------- forward pins

def _numpy_lowrank(d):
    x, A, B = _f64(d["x"]), _f64(d["A"]), _f64(d["B"])
    y = (x @ B.T) @ A.T
    if d["bias"] is not None:
        y = y + _f64(d["bias"])[None, :]
    return y


def _numpy_residual(d):
    x = _f64(d["x"])
    y = d["scale"] * (x @ _torch_dec(d["Q"]).T)
    if d["bias"] is not None:
        y = y + _f64(d["bias"])[None, :]
    return y


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def check_lowrank_only(lib):
    d = wl.random_inputs(9, 48, 40, 5, seed=1)
    d["Q"] = torch.zeros_like(d["Q"])
    y = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
    assert _rel(y, _numpy_lowrank(d)) < 1e-12


def check_residual_only(lib):
    d = wl.random_inputs(7, 64, 33, 4, seed=2)
    d["A"] = torch.zeros_like(d["A"])
    d["B"] = torch.zeros_like(d["B"])
    y = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
    assert _rel(y, _numpy_residual(d)) < 1e-12


def check_r0(lib):
    d = wl.random_inputs(5, 32, 17, 0, seed=3)
    y = oracle.forward(d["x"], None, None, d["Q"], d["scale"], d["bias"], lib=lib)
    assert _rel(y, _numpy_residual(d)) < 1e-12


def check_dense_equivalence(lib):
    for (M, K, N, r, seed) in [(4, 16, 8, 2, 4), (11, 80, 24, 7, 5), (3, 32, 64, 16, 6)]:
        d = wl.random_inputs(M, K, N, r, seed=seed)
        W = _f64(d["A"]) @ _f64(d["B"]) + d["scale"] * _torch_dec(d["Q"])
        ref = _f64(d["x"]) @ W.T + _f64(d["bias"])[None, :]
        y = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
        assert _rel(y, ref) < 1e-12, (M, K, N, r)


def _exact_forward(d):
    """Exact rational forward by pure-Python loops (tiny inputs only)."""
    fx = lambda t: [[Fraction(float(v)) for v in row] for row in t.to(torch.float64).tolist()]
    x, A, B = fx(d["x"]), fx(d["A"]), fx(d["B"])
    Qv = [[Fraction(float(v)) for v in row] for row in _torch_dec(d["Q"]).tolist()]
    s = Fraction(d["scale"])
    bias = [Fraction(float(v)) for v in d["bias"].to(torch.float64).tolist()]
    M, K, N, r = d["M"], d["in"], d["out"], d["r"]
    y = []
    for m in range(M):
        T = [sum(x[m][j] * B[k][j] for j in range(K)) for k in range(r)]
        y.append([sum(T[k] * A[n][k] for k in range(r)) + s * sum(x[m][j] * Qv[n][j] for j in range(K)) + bias[n]
                  for n in range(N)])
    return y


def check_bruteforce_rational(lib):
    d = wl.random_inputs(3, 16, 6, 3, seed=7)
    exact = _exact_forward(d)
    y = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
    for m in range(d["M"]):
        for n in range(d["out"]):
            e = float(exact[m][n])
            assert abs(y[m, n] - e) <= 1e-14 * max(abs(e), 1e-3), (m, n, y[m, n], e)


def check_exact_integer(lib):
    d = wl.exact_inputs(13, 96, 20, 6, seed=8)
    xi = d["x"].to(torch.int64).numpy()
    Ai = d["A"].to(torch.int64).numpy()
    Bi = d["B"].to(torch.int64).numpy()
    qi = _torch_dec(d["Q"]).astype(np.int64)
    b4 = (d["bias"].to(torch.float64).numpy() * 4).astype(np.int64)
    # 4*y = 4*T A^T + (x q^T) + 4*bias, with scale = 1/4
    y4 = 4 * ((xi @ Bi.T) @ Ai.T) + xi @ qi.T + b4[None, :]
    y = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
    assert np.array_equal(y * 4, y4.astype(np.float64))


def check_invariants(lib):
    d = wl.exact_inputs(6, 64, 12, 4, seed=9)
    fwd = lambda x, s=d["scale"], bias=d["bias"]: oracle.forward(x, d["A"], d["B"], d["Q"], s, bias, lib=lib)
    b = _f64(d["bias"])[None, :]
    x1 = d["x"]
    x2 = torch.roll(d["x"], 1, dims=1)
    lin = fwd(x1 + x2) - b
    assert np.array_equal(lin, (fwd(x1) - b) + (fwd(x2) - b))
    assert np.array_equal(fwd(x1, bias=None) + b, fwd(x1))
    y_res1 = fwd(x1, bias=None) - oracle.forward(x1, d["A"], d["B"], torch.zeros_like(d["Q"]), d["scale"], None, lib=lib)
    y_res2 = fwd(x1, s=2 * d["scale"], bias=None) - oracle.forward(x1, d["A"], d["B"], torch.zeros_like(d["Q"]), d["scale"], None, lib=lib)
    assert np.array_equal(2 * y_res1, y_res2)
    perm = torch.randperm(d["M"], generator=torch.Generator().manual_seed(0))
    assert np.array_equal(fwd(x1[perm]), fwd(x1)[perm.numpy()])
    rows = [5, 0, 3]
    assert np.array_equal(oracle.forward(x1, d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows, lib=lib),
                          fwd(x1)[rows])


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_hand_example():
    """The hand-worked forward in tests/golden/hand_example.json as tensors."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    codes = np.array([[int(c, 16) for c in row] for row in g["Q_codes_hex"]], dtype=np.uint8)
    d = {
        "x": torch.tensor(g["x"], dtype=torch.float32).to(torch.bfloat16),
        "A": torch.tensor(g["A"], dtype=torch.float32).to(torch.bfloat16),
        "B": torch.tensor(g["B"], dtype=torch.float32).to(torch.bfloat16),
        "Q": torch.from_numpy(codes),
        "scale": float(g["scale"]),
        "bias": torch.tensor(g["bias"], dtype=torch.float32).to(torch.bfloat16),
        "M": g["M"], "in": g["in"], "out": g["out"], "r": g["r"],
    }
    return d, np.array(g["y"], dtype=np.float64), g


def check_hand_example(lib):
    d, y_hand, g = load_hand_example()
    # the inputs are exact in bf16, and the code table matches the fixture's values
    assert np.array_equal(_f64(d["x"]), np.array(g["x"], np.float64))
    for code, v in g["Q_values"].items():
        assert lib.oracle_e4m3fn_to_f64(int(code, 16)) == v, code
    y = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], lib=lib)
    assert np.array_equal(y, y_hand), (y, y_hand)


PINS = [check_decode_vs_torch, check_lowrank_only, check_residual_only, check_r0,
        check_dense_equivalence, check_bruteforce_rational, check_exact_integer, check_invariants,
        check_hand_example]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_threads_do_not_change_result(oracle_lib):
    d = wl.random_inputs(33, 64, 40, 8, seed=10)
    a = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], threads=1, lib=oracle_lib)
    b = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], threads=4, lib=oracle_lib)
    assert np.array_equal(a, b)


def test_rejects_bad_rows(oracle_lib):
    d = wl.random_inputs(4, 16, 8, 2, seed=11)
    with pytest.raises(ValueError):
        oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=[4], lib=oracle_lib)


# Each planted mistake in litelinear_oracle.c (ORACLE_PLANT=n) must be caught.
PLANTS = {1: "bias dropped", 2: "scale ignored", 3: "subnormal sign lost",
          4: "exponent bias off by one", 5: "A transposed", 6: "B transposed",
          7: "low-rank term dropped"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p].replace(" ", "_"))
def test_planted_mistake_is_caught(plant):
    with tempfile.TemporaryDirectory() as td:
        path = oracle_build.build(os.path.join(td, f"liboracle_plant{plant}.so"), plant=plant)
        lib = oracle.library(path)
        caught = []
        for pin in PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin catches planted mistake {plant}: {PLANTS[plant]}"
