"""GPU parity of the decomposition side (litelinear_quantize_tensor,
litelinear_residual_quantize) against the float64 oracle, and properties of
the from_dense helper.

* The per-tensor quantiser of a given float32 array is bit-exact: same
  scale, same codes.
* The residual R = W - A B is summed in float32 on the GPU and in float64 by
  the oracle, so a code may differ where R / s sits within rounding of a
  boundary between two e4m3fn values: the scale must agree to 2 ulp, every
  code must be the oracle's or an adjacent one, and at most 1e-3 of them may
  differ.  Where A B is exact in float32 (r = 0, or small integers) the codes
  must agree bit for bit.
* from_dense (torch's SVD, then these kernels): A B is as close to W as the
  rank-r SVD allows (bf16 rounding aside), and A B + s dec(Q) rebuilds W to
  within half an e4m3fn step of the residual (computed here with torch).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Handle, Kernel, LiteLinearError, Option, Status
from rank_fp8_residual_amd import convert
from tests.test_oracle_convert_pins import quant_arrays

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


@pytest.mark.parametrize("case", range(len(quant_arrays()) + 1))
def test_quantize_tensor_bit_exact(dev, case):
    arrs = quant_arrays() + [np.random.default_rng(8).standard_normal(1 << 22).astype(np.float32) * 3e-3]
    R = arrs[case]
    R = R[: (R.size // 4) * 4] if R.size >= 4 else np.pad(R, (0, 4 - R.size))
    say("quantize_tensor", case, R.size)
    c_ref, s_ref = oracle.quantize_tensor(R)
    codes, scale = Handle(dev.index).quantize_tensor(torch.from_numpy(np.ascontiguousarray(R)).to(dev))
    torch.cuda.synchronize()
    assert float(scale.item()) == s_ref
    c = codes.cpu().numpy()
    bad = np.nonzero(c != c_ref)[0]
    assert bad.size == 0, (R[bad[:5]], c[bad[:5]], c_ref[bad[:5]])


def test_quantize_tensor_max_in_every_lane(dev):
    """The first pass reduces max |R| per wave (64 lanes) and work-group: a
    single largest value placed in each lane of the first and last wave of
    one work-group (four values per lane) sets the scale every time."""
    n = 3 * 256 * 4  # three work-groups of 256 threads, four values each
    base = np.random.default_rng(11).standard_normal(n).astype(np.float32) * 0.01
    h = Handle(dev.index)
    say("quantize_tensor max in every lane")
    for wave in (0, 3):
        for lane in range(64):
            R = base.copy()
            i = (256 + 64 * wave + lane) * 4 + lane % 4  # work-group 1
            R[i] = -7.5 if lane % 2 else 7.5
            c_ref, s_ref = oracle.quantize_tensor(R)
            codes, scale = h.quantize_tensor(torch.from_numpy(R).to(dev))
            torch.cuda.synchronize()
            assert float(scale.item()) == s_ref, (wave, lane)
            assert np.array_equal(codes.cpu().numpy(), c_ref), (wave, lane)


def _inputs(out, K, r, seed, exact=False):
    g = torch.Generator().manual_seed(seed)
    if exact:
        W = torch.randint(-8, 9, (out, K), generator=g).float()
        A = torch.randint(-2, 3, (out, r), generator=g).float()
        B = torch.randint(-2, 3, (r, K), generator=g).float()
    else:
        W = torch.randn(out, K, generator=g) * 0.05
        A = torch.randn(out, r, generator=g) * (0.05 / max(r, 1) ** 0.5)
        B = torch.randn(r, K, generator=g)
    return W.to(torch.bfloat16), A.to(torch.bfloat16), B.to(torch.bfloat16)


def _neighbours(c: np.ndarray, c_ref: np.ndarray) -> np.ndarray:
    """True where two e4m3fn codes are equal or adjacent on the value line."""
    def line(x):  # monotone index over the finite codes: -126..126
        x = x.astype(np.int64)
        return np.where(x & 0x80, -(x & 0x7F), x)
    return np.abs(line(c) - line(c_ref)) <= 1


RESID_SHAPES = [(40, 96, 16), (300, 512, 64), (257, 1040, 8), (1000, 2048, 64), (128, 256, 0), (700, 768, 512)]


@pytest.mark.parametrize("shape", RESID_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_residual_quantize_parity(dev, shape):
    out, K, r = shape
    W, A, B = _inputs(out, K, r, seed=out + K + r)
    say("residual_quantize", shape)
    R = oracle.residual(W, A, B) if r else W.double().numpy()
    c_ref, s_ref = oracle.quantize_tensor(R.astype(np.float32))
    h = Handle(dev.index)
    codes, scale = h.residual_quantize(W.to(dev), A.to(dev) if r else None, B.to(dev) if r else None)
    torch.cuda.synchronize()
    s = float(scale.item())
    c = codes.cpu().numpy()
    if r == 0:  # R = W exactly: bit-exact
        assert s == s_ref and np.array_equal(c, c_ref)
        return
    assert abs(s - s_ref) <= 2 * np.spacing(np.float32(s_ref)), (s, s_ref)
    assert np.all(_neighbours(c, c_ref)), np.argwhere(~_neighbours(c, c_ref))[:5]
    assert np.mean(c != c_ref) <= 1e-3, np.mean(c != c_ref)


def test_residual_quantize_max_in_last_of_many_tiles(dev):
    """More 128 x 128 tiles (65 x 64) than the second pass requests slots
    ahead for (4096): the largest |R| sits in the last tile, whose slot only
    the remainder loop reads."""
    out, K, r = 8320, 8192, 8
    W, A, B = _inputs(out, K, r, seed=41)
    W[-1, -1] = 8.0
    say("residual_quantize", (out, K, r), "max in the last tile")
    R = oracle.residual(W, A, B)
    c_ref, s_ref = oracle.quantize_tensor(R.astype(np.float32))
    codes, scale = Handle(dev.index).residual_quantize(W.to(dev), A.to(dev), B.to(dev))
    torch.cuda.synchronize()
    s = float(scale.item())
    assert abs(s - s_ref) <= 2 * np.spacing(np.float32(s_ref)), (s, s_ref)
    c = codes.cpu().numpy()
    assert np.all(_neighbours(c, c_ref))
    assert np.mean(c != c_ref) <= 1e-3


def test_residual_quantize_exact_products_bit_exact(dev):
    W, A, B = _inputs(300, 512, 32, seed=5, exact=True)
    R = oracle.residual(W, A, B)
    assert np.array_equal(R, np.round(R))  # integers: every float32 sum is exact
    c_ref, s_ref = oracle.quantize_tensor(R.astype(np.float32))
    say("residual_quantize exact")
    codes, scale = Handle(dev.index).residual_quantize(W.to(dev), A.to(dev), B.to(dev))
    torch.cuda.synchronize()
    assert float(scale.item()) == s_ref
    assert np.array_equal(codes.cpu().numpy(), c_ref)


@pytest.mark.parametrize("shape", [(512, 256, 32), (1024, 2048, 64)], ids=lambda s: "x".join(map(str, s)))
def test_from_dense_properties(dev, shape):
    out, K, r = shape
    g = torch.Generator().manual_seed(out + r)
    # a weight with a decaying spectrum, as trained layers have
    n = min(out, K)
    U = torch.linalg.qr(torch.randn(out, n, generator=g))[0]
    V = torch.linalg.qr(torch.randn(K, n, generator=g))[0]
    sv = torch.exp(-torch.arange(n, dtype=torch.float32) / (n / 8))
    W = ((U * sv) @ V.T * 0.5).to(torch.bfloat16)
    say("from_dense", shape)
    f = convert.from_dense(W.to(dev), r)
    torch.cuda.synchronize()
    A, B, Q, s = f["A"].float().cpu(), f["B"].float().cpu(), f["Q"].cpu(), float(f["scale"].item())
    Wf = W.double()
    AB = A.double() @ B.double()
    # rank-r optimum (Eckart-Young) from the singular values of the bf16 W
    svals = torch.linalg.svdvals(Wf)
    opt = float(torch.sqrt((svals[r:] ** 2).sum()))
    err = float(torch.linalg.norm(Wf - AB))
    assert err <= opt * 1.02 + 2.0 ** -8 * float(torch.linalg.norm(Wf)), (err, opt)
    # A B + s dec(Q) rebuilds W within half an e4m3fn step of R
    R = Wf - AB
    dec = Q.view(torch.float8_e4m3fn).double() * s
    step = torch.maximum(R.abs() * 2.0 ** -4, torch.full_like(R, s * 2.0 ** -10))
    # (the kernel rounds a float32 R, which sits within ~2^-24 |W| of this one)
    assert bool(((R - dec).abs() <= step * 1.001 + 2.0 ** -20 * float(Wf.abs().max())).all())
    assert abs(s - float(R.abs().max()) / 448.0) <= 1e-5 * s


def test_convert_errors(dev):
    h = Handle(dev.index)
    say("convert errors")
    W = torch.zeros((64, 96), dtype=torch.bfloat16, device=dev)
    A = torch.zeros((64, 12), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((12, 96), dtype=torch.bfloat16, device=dev)
    with pytest.raises(LiteLinearError) as e:  # r % 8 != 0
        h.residual_quantize(W, A, B)
    assert e.value.status == Status.UNSUPPORTED
    with pytest.raises(LiteLinearError) as e:  # n % 4 != 0
        h.quantize_tensor(torch.zeros(6, dtype=torch.float32, device=dev))
    assert e.value.status == Status.UNSUPPORTED
    h.set_option(Option.PROFILE, 1)
    c, s = h.residual_quantize(W, None, None)
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and bool((c == 0).all())  # all-zero R: scale 1, codes +0
    assert h.kernel_time(Kernel.CONVERT)[1] == 1
