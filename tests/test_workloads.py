"""The seeded input generator: shapes, dtypes, determinism and the quantiser's
saturation (data generation only; no forward arithmetic here)."""
import numpy as np
import pytest
import torch

from rank_fp8_residual_amd import workloads as wl


def test_shapes_and_dtypes():
    d = wl.make_inputs("tiny")
    assert d["x"].shape == (64, 256) and d["x"].dtype == torch.bfloat16
    assert d["A"].shape == (256, 16) and d["B"].shape == (16, 256)
    assert d["Q"].shape == (256, 256) and d["Q"].dtype == torch.uint8
    assert d["bias"].shape == (256,) and isinstance(d["scale"], float)


def test_seeded_and_deterministic():
    a, b = wl.make_inputs("tiny", seed=3), wl.make_inputs("tiny", seed=3)
    c = wl.make_inputs("tiny", seed=4)
    assert all(torch.equal(a[k], b[k]) for k in ("x", "A", "B", "Q", "bias"))
    assert not torch.equal(a["x"], c["x"])


def test_quantiser_saturates_and_never_makes_nan():
    R = torch.tensor([[-1000.0, -448.0, -1e-9, 0.0, 1e-9, 300.0, 448.0, 464.0, 480.0, 1e6]])
    q = wl.quantize_e4m3fn(R)[0]
    vals = q.view(torch.float8_e4m3fn).to(torch.float32)
    assert torch.isfinite(vals).all()
    assert not ((q == 0x7F) | (q == 0xFF)).any()
    s = float(np.float32(1e6 / 448))
    assert vals.abs().max().item() == 448.0
    assert wl.quantize_e4m3fn(R)[1] == s


def test_scale_is_amax_over_448():
    d = wl.make_inputs("tiny")
    codes = d["Q"].view(torch.float8_e4m3fn).to(torch.float32)
    assert codes.abs().max().item() == 448.0   # the largest |R| maps to the largest code
    assert 0.02 * 3 / 448 < d["scale"] < 0.02 * 6 / 448


def test_dit_outlier_channels():
    d = wl.make_inputs(wl.Workload("dit_small", 512, 2048, 64, 8, outlier_frac=0.01), seed=0)
    col_rms = d["x"].to(torch.float32).pow(2).mean(0).sqrt()
    assert int((col_rms > 5).sum()) == 20   # round(0.01 * 2048) channels scaled by 20


def test_exact_inputs_bounds():
    d = wl.exact_inputs(8, 512, 16, 8)
    T = d["x"].to(torch.float64) @ d["B"].to(torch.float64).T
    assert T.abs().max() <= 256
    assert int((d["B"] != 0).sum(1).max()) <= 64


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_workload_sizes(name):
    w = wl.WORKLOADS[name]
    assert w.flops == 2 * w.M * (w.in_features * w.out_features + w.rank * (w.in_features + w.out_features))
    assert w.bytes > w.in_features * w.out_features
