"""GPU parity of the input and epilogue variants against the float64 oracle.

* e4m3fnuz residual codes (LITELINEAR_OPT_Q_FORMAT = 1, the format the
  LiteLinear README's Features list names for AMD hardware): every code
  decodes exactly (identity activations, float32 output, bit for bit), the
  +-240 codes that a per-tensor quantiser puts at the largest magnitude and
  the NaN code 0x80 included; random and full-size forwards meet the bf16
  gates against the oracle's e4m3fnuz forward.
* GEGLU (LITELINEAR_OPT_ACTIVATION = 2; the README's integration guide
  passes a GEGLU's activation projection through LiteLinear): y = hidden *
  GELU(gate) over the halves of the 2F-row projection, against
  oracle.geglu of the oracle's forward.  Gate: the forward's own error
  bound eps = 2e-2 RMS(v) on both halves, carried through the product
  (|dy| <= eps (|GELU(g)| + 1.13 |h| + 1.13 eps), 1.13 bounding the exact
  GELU's slope), plus half a bf16 ulp for the output's rounding, and
  relative L1 <= 5e-3.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Activation, Handle, LiteLinearError, Option, Path, Status
from rank_fp8_residual_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu

PATHS = [Path.SKINNY, Path.TILED]


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def to_dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def handle(dev, path=Path.AUTO, out_f32=False, fnuz=False, geglu=False, act8=False):
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(path))
    h.set_option(Option.OUTPUT_F32, int(out_f32))
    h.set_option(Option.Q_FORMAT, int(fnuz))
    h.set_option(Option.ACTIVATION, int(Activation.GEGLU if geglu else Activation.NONE))
    h.set_option(Option.ACT_FP8, int(act8))
    return h


def fwd(h, g):
    y = h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    return y


def ref(d, rows=None, fnuz=False, act8=False):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"], d["scale"],
                          d["bias"], rows=rows, q_format="e4m3fnuz" if fnuz else "e4m3fn", act_fp8=act8)


# ------------------------------------------------------------------ e4m3fnuz

@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_fnuz_decode_every_code_bit_exact(dev, path):
    """x = identity: y = dec(Q) column by column, for all 255 non-NaN codes
    (+-240 among them, several per fragment), float32 output, bit for bit."""
    codes = np.array([c for c in range(256) if c != 0x80], np.uint8)
    K = 256
    Qn = np.zeros((16, K), np.uint8)
    for i in range(16):
        Qn[i] = np.roll(np.concatenate([codes, codes[:1]]), 13 * i)[:K]
    Qn[3, 5:9] = [0x7F, 0xFF, 0x7F, 0x01]  # exceptional codes side by side
    d = {"x": torch.eye(K, dtype=torch.bfloat16)[:64].contiguous(), "A": None, "B": None,
         "Q": torch.from_numpy(Qn), "scale": 1.0, "bias": None, "M": 64, "in": K, "out": 16, "r": 0}
    say("fnuz decode", path.name)
    y = parity.to_f64(fwd(handle(dev, path, out_f32=True, fnuz=True), to_dev(d, dev)))
    assert np.array_equal(y, oracle.decode_e4m3fnuz(Qn[:, :64]).T)


@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_fnuz_nan_code_propagates(dev, path):
    d = wl.random_inputs(16, 512, 320, 16, seed=600, q_format="e4m3fnuz")
    d["Q"][7, 100] = 0x80
    say("fnuz nan", path.name)
    y = parity.to_f64(fwd(handle(dev, path, fnuz=True), to_dev(d, dev)))
    assert np.all(np.isnan(y[:, 7]))
    assert np.all(np.isfinite(np.delete(y, 7, axis=1)))


FNUZ_SHAPES = [  # M, in, out, r
    (16, 2048, 1024, 64), (40, 512, 640, 32), (64, 256, 256, 16), (300, 1024, 520, 48),
    (2000, 512, 4000, 64), (1000, 768, 1030, 256),
]


@pytest.mark.parametrize("shape", FNUZ_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_fnuz_random_parity(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=610 + M, q_format="e4m3fnuz")
    q = d["Q"]
    assert bool(((q == 0x7F) | (q == 0xFF)).any())  # the largest magnitude sits on +-240
    y_ref = ref(d, fnuz=True)
    g = to_dev(d, dev)
    for path in PATHS:
        if path == Path.SKINNY and M > 64:
            continue
        say("fnuz random", shape, path.name, "f32" if out_f32 else "bf16")
        parity.check(parity.to_f64(fwd(handle(dev, path, out_f32, fnuz=True), g)), y_ref, out_f32)


def test_fnuz_many_exceptional_codes(dev):
    """Codes of +-240 scattered over every K step and column tile (so that
    each wave's fix-up runs often), against the oracle."""
    d = wl.random_inputs(1024, 1024, 2048, 64, seed=620, q_format="e4m3fnuz")
    gen = torch.Generator().manual_seed(621)
    mask = torch.rand(d["Q"].shape, generator=gen) < 0.002
    d["Q"][mask] = torch.where(torch.rand(int(mask.sum()), generator=gen) < 0.5, 0x7F, 0xFF).to(torch.uint8)
    say("fnuz many +-240", int(mask.sum()))
    for path in (Path.TILED,):
        parity.check(parity.to_f64(fwd(handle(dev, path, fnuz=True), to_dev(d, dev))), ref(d, fnuz=True), False)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["skinny", "dit_r64", "llm"])
def test_fnuz_workload_full_output(dev, name):
    w = wl.WORKLOADS[name]
    d = wl.make_inputs(w, seed=0, q_format="e4m3fnuz")
    say("fnuz workload", name)
    y = fwd(handle(dev, fnuz=True), to_dev(d, dev))
    m = parity.check_full(y, lambda rows: ref(d, rows=rows, fnuz=True), w.M, False)
    say("fnuz workload", name, {k: v for k, v in m.items() if k in ("max_over_rms", "rel_l1")})


def test_fnuz_with_fp8_activations_is_refused(dev):
    d = wl.random_inputs(300, 256, 256, 16, seed=630, q_format="e4m3fnuz")
    g = to_dev(d, dev)
    with pytest.raises(LiteLinearError) as ei:
        handle(dev, fnuz=True, act8=True).forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert ei.value.status == Status.UNSUPPORTED


# --------------------------------------------------------------------- GEGLU

def check_geglu(y, v_ref, out_f32):
    """y [rows, F] against GEGLU of the oracle's [rows, 2F] forward v_ref."""
    F = v_ref.shape[1] // 2
    h, gate = v_ref[:, :F], v_ref[:, F:]
    y_ref = oracle.geglu(v_ref)
    eps = parity.MAX_RMS_GATE * float(np.sqrt(np.mean(v_ref ** 2)))
    bound = eps * (np.abs(oracle.gelu_erf(gate)) + 1.13 * np.abs(h) + 1.13 * eps) + 1e-6 * np.abs(y_ref)
    if not out_f32:
        bound = bound + parity.half_ulp_bf16(y_ref)
    d = np.abs(y - y_ref)
    assert np.all(np.isfinite(y))
    bad = d > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3].tolist())
    l1 = float(d.sum() / np.abs(y_ref).sum())
    assert l1 <= parity.REL_L1_GATE, l1
    return {"max_abs": float(d.max()), "rel_l1": l1}


GEGLU_SHAPES = [  # M, in, out (= 2F), r
    (1, 256, 512, 16), (16, 2048, 2048, 64), (40, 512, 1040, 32), (64, 256, 256, 16), (300, 1024, 520, 48),
    (2000, 512, 4000, 64), (3630, 256, 8192, 64), (1000, 768, 1032, 256), (512, 512, 8192, 256),
    (4096, 256, 4096, 256),
]


@pytest.mark.parametrize("shape", GEGLU_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode", ["bf16", "f32", "act8", "fnuz"])
def test_geglu_parity(dev, shape, mode):
    M, K, N, r = shape
    fnuz, act8, out_f32 = mode == "fnuz", mode == "act8", mode == "f32"
    d = wl.random_inputs(M, K, N, r, seed=700 + M, q_format="e4m3fnuz" if fnuz else "e4m3fn")
    g = to_dev(d, dev)
    rows = np.arange(M) if M <= 512 else np.unique(np.linspace(0, M - 1, 300).astype(np.int64))
    v_ref = ref(d, rows=rows, fnuz=fnuz, act8=act8)
    for path in PATHS:
        if path == Path.SKINNY and (M > 64 or act8):
            continue
        say("geglu", shape, mode, path.name)
        y = fwd(handle(dev, path, out_f32, fnuz=fnuz, geglu=True, act8=act8), g)
        assert y.shape == (M, N // 2)
        check_geglu(parity.to_f64(y[torch.from_numpy(rows).to(dev)]), v_ref, out_f32)


@pytest.mark.timeout(600)
def test_geglu_dit_full_output(dev):
    """The DiT feed-forward input projection as a GEGLU: 3630 tokens, 2048 ->
    2 x 4096, rank 64, every output against the oracle."""
    w = wl.WORKLOADS["dit_r64"]
    d = wl.make_inputs(w, seed=0)
    say("geglu dit full")
    y = fwd(handle(dev, geglu=True), to_dev(d, dev))
    for m0 in range(0, w.M, 512):
        rows = np.arange(m0, min(w.M, m0 + 512))
        check_geglu(parity.to_f64(y[m0:m0 + 512]), ref(d, rows=rows), False)


def test_geglu_errors(dev):
    d = wl.random_inputs(300, 256, 257, 16, seed=720)  # odd out: no two halves
    g = to_dev(d, dev)
    h = handle(dev, geglu=True)
    with pytest.raises(LiteLinearError) as ei:
        h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert ei.value.status == Status.INVALID_ARG
    d = wl.random_inputs(300, 256, 256, 16, seed=721)
    g = to_dev(d, dev)
    with pytest.raises(LiteLinearError) as ei:
        h.forward_pair(g["x"], g["B"], (g["A"], g["Q"], g["scale"], g["bias"]),
                       (g["A"], g["Q"], g["scale"], g["bias"]))
    assert ei.value.status == Status.UNSUPPORTED
    with pytest.raises(LiteLinearError):
        h.set_option(Option.ACTIVATION, 3)
