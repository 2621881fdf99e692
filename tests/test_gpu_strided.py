"""x read with a row stride (litelinear_forward_strided): x is a row slice
of a wider tensor whose other columns hold NaN, so a read outside a row's
`in` elements would show in y.  The strided forward must equal the forward
on a contiguous copy of x bit for bit (the same kernels and arithmetic) and
meet the oracle's gates; the stride's argument errors are reported."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from rank_fp8_residual_amd import Option, Path, Status
from rank_fp8_residual_amd import litelinear as L
from rank_fp8_residual_amd import workloads as wl
from tests import parity
from tests.test_gpu_parity import make_handle, oracle_y, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def wide_copy(x: torch.Tensor, pad: int, dev) -> torch.Tensor:
    """x [M, in] as the first `in` columns of a [M, in + pad] device tensor
    whose other columns are NaN."""
    M, K = x.shape
    big = torch.full((M, K + pad), float("nan"), dtype=torch.bfloat16, device=dev)
    big[:, :K] = x.to(dev)
    return big[:, :K]


def fwd(h, d, x, dev):
    t = lambda v: v.to(dev) if isinstance(v, torch.Tensor) else v
    r = d["r"]
    y = h.forward(x, t(d["A"]) if r else None, t(d["B"]) if r else None, t(d["Q"]), d["scale"], t(d["bias"]))
    torch.cuda.synchronize()
    return y


CASES = [  # (M, in, out, r), path, pad
    ((16, 2048, 1030, 64), Path.SKINNY, 8), ((40, 512, 512, 32), Path.AUTO, 64),
    ((64, 256, 256, 16), Path.AUTO, 24), ((300, 1024, 520, 48), Path.TILED, 8),
    ((1000, 768, 1030, 256), Path.TILED, 256), ((513, 512, 700, 0), Path.TILED, 16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[0])) + f"-{c[1].name}-pad{c[2]}")
def test_strided_x_matches_contiguous(dev, case):
    (M, K, N, r), path, pad = case
    d = wl.random_inputs(M, K, N, r, seed=600 + M)
    say("strided", (M, K, N, r), path.name, "pad", pad)
    h = make_handle(dev, path)
    xs = wide_copy(d["x"], pad, dev)
    assert not xs.is_contiguous() and xs.stride(0) == K + pad
    y_s = fwd(h, d, xs, dev)
    y_c = fwd(h, d, d["x"].to(dev), dev)
    assert torch.equal(y_s, y_c)
    parity.check(parity.to_f64(y_s), oracle_y(d), False)


def test_strided_x_256x256_tiles_and_act8(dev):
    M, K, N, r = 4096, 512, 4096, 64
    d = wl.random_inputs(M, K, N, r, seed=61)
    say("strided 256x256 + act8", (M, K, N, r))
    xs = wide_copy(d["x"], 64, dev)
    for act8 in (False, True):
        h = make_handle(dev, Path.TILED)
        h.set_option(Option.ACT_FP8, int(act8))
        y_s = fwd(h, d, xs, dev)
        y_c = fwd(h, d, d["x"].to(dev), dev)
        assert torch.equal(y_s, y_c), act8
    rows = sample_rows(M, 24)
    import oracle
    y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows, act_fp8=True)
    parity.check(parity.to_f64(y_s[torch.from_numpy(rows).to(dev)]), y_ref, False)


def test_three_dimensional_slice(dev):
    """x [2, 150, in] sliced from [2, 150, in + 40]: the leading dimensions
    flatten to rows of one stride."""
    B_, S, K, N, r = 2, 150, 512, 300, 32
    d = wl.random_inputs(B_ * S, K, N, r, seed=62)
    big = torch.full((B_, S, K + 40), float("nan"), dtype=torch.bfloat16, device=dev)
    big[..., :K] = d["x"].view(B_, S, K).to(dev)
    say("strided 3-d")
    h = make_handle(dev)
    y = fwd(h, d, big[..., :K], dev)
    assert y.shape == (B_, S, N)
    assert torch.equal(y.view(B_ * S, N), fwd(h, d, d["x"].to(dev), dev))


def test_stride_errors(dev):
    d = wl.random_inputs(32, 256, 64, 16, seed=63)
    h = make_handle(dev)
    say("strided errors")
    with pytest.raises(L.LiteLinearError) as e:  # rows not 16-byte aligned
        fwd(h, d, wide_copy(d["x"], 4, dev), dev)
    assert e.value.status == Status.UNSUPPORTED
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    y = torch.empty((32, 64), dtype=torch.bfloat16, device=dev)
    args = (g["A"].data_ptr(), g["B"].data_ptr(), g["Q"].data_ptr(), ctypes.c_float(g["scale"]),
            g["bias"].data_ptr(), y.data_ptr(), 32, 256, 64, 16, None)
    lib = L.lib()
    assert lib.litelinear_forward_strided(h._h, g["x"].data_ptr(), 240, *args) == Status.INVALID_ARG  # ldx < in
    assert lib.litelinear_forward_strided(h._h, g["x"].data_ptr(), 256, *args) == Status.OK
    torch.cuda.synchronize()
    assert torch.equal(y, fwd(h, d, g["x"], dev))
