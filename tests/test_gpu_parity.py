"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Every case prints its name, shape, path and seed before it touches the GPU.
Gates are in tests/parity.py.  Exact-arithmetic inputs must agree bit for
bit; the e4m3fn decode must be bit-exact for every code.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from rank_fp8_residual_amd import Handle, Kernel, LiteLinearError, Option, Path, Status
from rank_fp8_residual_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def to_dev(d, dev):
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    return g


def make_handle(dev, path=Path.AUTO, out_f32=False, split=0):
    h = Handle(dev.index)
    h.set_option(Option.PATH, int(path))
    h.set_option(Option.OUTPUT_F32, int(out_f32))
    h.set_option(Option.SPLIT_K, split)
    return h


def run(h, g):
    y = h.forward(g["x"], g["A"] if g["r"] else None, g["B"] if g["r"] else None, g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    return y


def oracle_y(d, rows=None):
    return oracle.forward(d["x"], d["A"] if d["r"] else None, d["B"] if d["r"] else None, d["Q"],
                          d["scale"], d["bias"], rows=rows)


PATHS = [Path.SKINNY, Path.TILED]


# ------------------------------------------------------------ exact decode

@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_decode_every_code_bit_exact(dev, path):
    """y = x dec(Q)^T with x = identity returns every e4m3fn value exactly."""
    say("decode", path.name)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    K = 256
    Qn = np.zeros((16, K), np.uint8)
    for i in range(16):
        Qn[i] = np.roll(np.concatenate([codes, codes[:2]]), 17 * i)[:K]
    d = {"x": torch.eye(K, dtype=torch.bfloat16)[:64].contiguous(), "A": None, "B": None,
         "Q": torch.from_numpy(Qn), "scale": 1.0, "bias": None, "M": 64, "in": K, "out": 16, "r": 0}
    h = make_handle(dev, path, out_f32=True)
    y = parity.to_f64(run(h, to_dev(d, dev)))
    expect = oracle.decode_e4m3fn(Qn[:, :64]).T
    assert np.array_equal(y, expect)  # -0 == +0: a sum cannot keep the sign of a zero


# ------------------------------------------------------ hand example

@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_hand_example(dev, path):
    """The forward worked by hand in tests/golden/hand_example.json: float32
    output must equal it exactly, bf16 output must be its nearest-even bf16."""
    from tests.test_oracle_pins import load_hand_example
    d, y_hand, _ = load_hand_example()
    g = to_dev(d, dev)
    say("hand example", path.name)
    y32 = parity.to_f64(run(make_handle(dev, path, out_f32=True), g))
    assert np.array_equal(y32, y_hand), (y32, y_hand)
    y16 = parity.to_f64(run(make_handle(dev, path), g))
    assert np.array_equal(y16, parity.bf16_of(y_hand)), (y16, y_hand)


# ------------------------------------------------------- exact arithmetic

EXACT_SHAPES = [  # M, in, out, r
    (1, 16, 5, 0), (7, 48, 17, 3), (16, 64, 256, 16), (33, 320, 200, 17), (64, 256, 260, 64),
    (67, 96, 129, 1), (130, 64, 300, 100), (257, 512, 513, 64), (300, 2048, 64, 128),
]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_exact_inputs_bitwise(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.exact_inputs(M, K, N, r, seed=M + K + N + r)
    y_ref = oracle_y(d)
    expect = y_ref if out_f32 else parity.bf16_of(y_ref)
    g = to_dev(d, dev)
    for path in PATHS:
        if path == Path.SKINNY and M > 64:
            continue
        say("exact", shape, path.name, "f32" if out_f32 else "bf16")
        y = parity.to_f64(run(make_handle(dev, path, out_f32), g))
        bad = np.argwhere(y != expect)
        assert bad.size == 0, (path.name, bad[:5].tolist(), y[tuple(bad[0])], expect[tuple(bad[0])])


EXACT_GRID_SHAPES = [  # M, in, out, r: the tile sizes and T producers of the full-size workloads
    (4096, 256, 4096, 64),    # 256 x 256 tiles (ping-pong loop), two 128-row T blocks per row tile
    (4096, 128, 4096, 256),   # 256 x 256 tiles, 256-column T blocks
    (3630, 192, 8192, 64),    # the DiT grid: 480 tiles of 256 x 256, a 46-row last row tile
    (2048, 256, 4096, 64),    # 256 x 128 tiles (lockstep loop), two 128-row T blocks
    (2000, 320, 4000, 48),    # 256 x 128 tiles with ragged rows, columns and rank
]


@pytest.mark.parametrize("shape", EXACT_GRID_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_inputs_bitwise_large_tiles(dev, shape):
    """Exact-arithmetic inputs on grids that select the 256 x 256 and
    256 x 128 tiles: bf16 and float32 outputs equal the oracle bit for bit,
    on the automatic path and on two calls with different inputs queued back
    to back on one handle."""
    M, K, N, r = shape
    h16, h32 = make_handle(dev, Path.AUTO), make_handle(dev, Path.AUTO, out_f32=True)
    ds = [wl.exact_inputs(M, K, N, r, seed=s) for s in (M + r, M + r + 1)]
    gs = [to_dev(d, dev) for d in ds]
    say("exact large tiles", shape)
    ys = [(h16.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"]),
           h32.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])) for g in gs]
    torch.cuda.synchronize()
    for d, (y16, y32) in zip(ds, ys):
        y_ref = oracle_y(d)
        for y, expect in ((y32, y_ref), (y16, parity.bf16_of(y_ref))):
            y = parity.to_f64(y)
            bad = np.argwhere(y != expect)
            assert bad.size == 0, (bad[:5].tolist(), y[tuple(bad[0])], expect[tuple(bad[0])])


# --------------------------------------------------- random small shapes

RANDOM_SHAPES = [  # M, in, out, r: several tiles and ragged tails
    (1, 256, 300, 16), (16, 1024, 777, 64), (40, 512, 512, 32), (64, 2048, 1024, 64),
    (65, 256, 256, 16), (200, 1024, 520, 48), (513, 512, 700, 64), (1000, 768, 1030, 256),
]


@pytest.mark.parametrize("shape", RANDOM_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16", "f32"])
def test_random_parity(dev, shape, out_f32):
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=1000 + M)
    y_ref = oracle_y(d)
    g = to_dev(d, dev)
    for path in PATHS:
        if path == Path.SKINNY and M > 64:
            continue
        say("random", shape, path.name, "f32" if out_f32 else "bf16")
        y = parity.to_f64(run(make_handle(dev, path, out_f32), g))
        parity.check(y, y_ref, out_f32)


@pytest.mark.parametrize("t_splits", [1, 2, 3, 5, 0])
def test_tiled_t_split_counts(dev, t_splits):
    """T = x B^T summed over K slices: same gates, and repeat calls agree bit
    for bit (the slice counters are back at zero, the sum order is fixed)."""
    d = wl.random_inputs(300, 1280, 520, 80, seed=17)
    y_ref = oracle_y(d)
    say("tiled t_splits", t_splits)
    h = make_handle(dev, Path.TILED)
    h.set_option(Option.T_SPLITS, t_splits)
    g = to_dev(d, dev)
    y1 = run(h, g)
    y2 = run(h, g)
    assert torch.equal(y1, y2)
    parity.check(parity.to_f64(y1), y_ref, False)


@pytest.mark.parametrize("shape", [(512, 1024, 8192, 64), (890, 768, 4600, 40), (4096, 512, 4096, 256)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("act8", [False, True], ids=["bf16", "act8"])
def test_tiled_full_round_grids(dev, shape, act8):
    """Output grids of one full round of work-groups (or nearly), so that the
    T producers push output tiles into a second round (64- and 256-column T
    blocks); checked on sampled rows, and repeat calls agree bit for bit."""
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=80 + r)
    say("tiled full round", shape, "act8" if act8 else "bf16")
    h = make_handle(dev, Path.TILED)
    h.set_option(Option.ACT_FP8, int(act8))
    g = to_dev(d, dev)
    y1 = run(h, g)
    y2 = run(h, g)
    assert torch.equal(y1, y2)
    rows = sample_rows(M, 40)
    y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows, act_fp8=act8)
    parity.check(parity.to_f64(y1[torch.from_numpy(rows).to(dev)]), y_ref, False)


@pytest.mark.parametrize("shape", [(2000, 1008, 4000, 48), (2304, 2064, 3968, 64), (2048, 48, 4096, 16),
                                   (1800, 16, 4100, 8), (2048, 4096, 4096, 64)], ids=lambda s: "x".join(map(str, s)))
def test_tiled_256x128_tiles(dev, shape):
    """Grids of 256 x 128 output tiles (at least 256 of them, fewer than 256
    of 256 x 256): K ends 16 or 48 elements into a 64-element step, or on
    one (for in = 16 and 48 the only step is that partial one), with ragged
    row and column tiles; sampled rows of every row tile, and repeat calls
    agree bit for bit."""
    M, K, N, r = shape
    assert -(-M // 256) * -(-N // 128) >= 256 > -(-M // 256) * -(-N // 256)
    d = wl.random_inputs(M, K, N, r, seed=90 + r)
    say("tiled 256x128", shape)
    h = make_handle(dev, Path.TILED)
    g = to_dev(d, dev)
    y1 = run(h, g)
    y2 = run(h, g)
    assert torch.equal(y1, y2)
    rows = sample_rows(M, 40)
    y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], rows=rows)
    parity.check(parity.to_f64(y1[torch.from_numpy(rows).to(dev)]), y_ref, False)


TINY_SHAPES = [(64, 256, 256, 16), (100, 128, 300, 100), (40, 64, 520, 64), (257, 256, 48, 8)]


@pytest.mark.parametrize("shape", TINY_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mode", ["bf16", "f32", "unfolded", "act8"])
def test_tiled_tiny_problems_compute_t_in_each_tile(dev, shape, mode):
    """Tiny problems (in <= 256, M in (32, ...], M in out <= 2^22): the output
    tiles compute T themselves (one or two 64-rank blocks), on the automatic
    path as well as the forced tiled one; repeat calls agree bit for bit."""
    M, K, N, r = shape
    d = wl.random_inputs(M, K, N, r, seed=90 + M)
    if mode == "unfolded":
        d["scale"] = 2.0 ** -70
    act8 = mode == "act8"
    y_ref = oracle.forward(d["x"], d["A"], d["B"], d["Q"], d["scale"], d["bias"], act_fp8=act8)
    g = to_dev(d, dev)
    for path in (Path.AUTO, Path.TILED):
        say("tiny tiled", shape, mode, path.name)
        h = make_handle(dev, path, out_f32=mode in ("f32", "unfolded"))
        h.set_option(Option.ACT_FP8, int(act8))
        y1 = run(h, g)
        assert torch.equal(y1, run(h, g))
        parity.check(parity.to_f64(y1), y_ref, mode in ("f32", "unfolded"))


def test_tiled_tiny_pair(dev):
    d1 = wl.random_inputs(64, 256, 200, 48, seed=95)
    d2 = wl.random_inputs(64, 256, 136, 48, seed=96)
    d2["x"], d2["B"], d2["scale"] = d1["x"], d1["B"], d1["scale"] * 3.0
    g1, g2 = to_dev(d1, dev), to_dev(d2, dev)
    say("tiny tiled pair")
    h = make_handle(dev, Path.TILED)
    y1, y2 = h.forward_pair(g1["x"], g1["B"], (g1["A"], g1["Q"], g1["scale"], g1["bias"]),
                            (g2["A"], g2["Q"], g2["scale"], g2["bias"]))
    torch.cuda.synchronize()
    parity.check(parity.to_f64(y1), oracle_y(d1), False)
    parity.check(parity.to_f64(y2), oracle_y(d2), False)


@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_bf16_output_is_rne_of_f32_output(dev, path):
    """The bf16 output is the float32 output rounded to nearest even (the
    kernels accumulate identically in both modes; only the final store
    differs), checked element by element, including values placed exactly
    halfway between bf16 neighbours, subnormal-range and huge results."""
    M = 48 if path == Path.SKINNY else 300
    d = wl.random_inputs(M, 512, 640, 32, seed=71)
    g = to_dev(d, dev)
    say("bf16 rounding", path.name)
    y32 = run(make_handle(dev, path, out_f32=True), g)
    y16 = run(make_handle(dev, path), g)
    assert torch.equal(y32.to(torch.bfloat16), y16)
    # halfway cases: scale the same inputs by powers of two so results span the
    # bf16 range, and use exact inputs whose sums land on ties
    for sc in (2.0 ** -120, 2.0 ** 100):
        g2 = dict(g, scale=g["scale"] * sc, A=g["A"] * 0, bias=None)
        y32 = run(make_handle(dev, path, out_f32=True), g2)
        y16 = run(make_handle(dev, path), g2)
        assert torch.equal(y32.to(torch.bfloat16), y16), sc
    de = wl.exact_inputs(M, 512, 640, 16, seed=72)
    ge = to_dev(de, dev)
    y32 = run(make_handle(dev, path, out_f32=True), ge)
    y16 = run(make_handle(dev, path), ge)
    assert torch.equal(y32.to(torch.bfloat16), y16)


@pytest.mark.parametrize("r", [256, 512, 320])
def test_wide_t_blocks(dev, r):
    """Ranks that are multiples of 256 on 256 x 256 output tiles take T in
    256-column producer blocks (320 does not, for comparison); sampled rows
    against the oracle, bf16 and float32 output."""
    M, K, N = 4096, 512, 4096
    d = wl.random_inputs(M, K, N, r, seed=60 + r)
    g = to_dev(d, dev)
    rows = sample_rows(M, 40)
    y_ref = oracle_y(d, rows=rows)
    for out_f32 in (False, True):
        say("wide T blocks", r, "f32" if out_f32 else "bf16")
        y = run(make_handle(dev, Path.TILED, out_f32), g)
        parity.check(parity.to_f64(y[torch.from_numpy(rows).to(dev)]), y_ref, out_f32)


@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_handle_reuse_across_shapes(dev, path):
    """One handle, a sequence of shapes that change the column-tile count,
    the row-tile count, the rank (and so the T flag step), with r = 0 calls
    and tiny problems (T computed in each output tile, counters untouched) in
    between: every call must match the oracle (the handle's counters are
    restarted whenever their layout changes)."""
    if path == Path.SKINNY:
        shapes = [(16, 512, 256, 64), (16, 512, 1024, 64), (16, 512, 1024, 0), (16, 512, 256, 64),
                  (16, 512, 256, 128), (9, 1024, 2176, 64), (16, 512, 256, 64)]
    else:
        shapes = [(300, 256, 512, 64), (300, 128, 100, 64), (600, 256, 512, 64), (300, 256, 512, 128),
                  (300, 256, 512, 0), (64, 256, 256, 16), (300, 256, 512, 64), (700, 512, 384, 192),
                  (300, 128, 100, 64), (300, 256, 512, 64)]
    h = make_handle(dev, path)
    cache = {}
    for rep in range(2):
        for i, (M, K, N, r) in enumerate(shapes):
            say("reuse", path.name, rep, (M, K, N, r))
            if (M, K, N, r) not in cache:
                d = wl.random_inputs(M, K, N, r, seed=40 + i)
                cache[(M, K, N, r)] = (d, oracle_y(d), to_dev(d, dev))
            d, y_ref, g = cache[(M, K, N, r)]
            parity.check(parity.to_f64(run(h, g)), y_ref, False)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 32])
def test_skinny_split_counts(dev, splits):
    d = wl.random_inputs(16, 2048, 640, 64, seed=7)
    y_ref = oracle_y(d)
    say("skinny splits", splits)
    h = make_handle(dev, Path.SKINNY, split=splits)
    g = to_dev(d, dev)
    y1 = run(h, g)
    y2 = run(h, g)  # the counters must be back at zero for the second call
    assert torch.equal(y1, y2)
    parity.check(parity.to_f64(y1), y_ref, False)


# ------------------------------------------------------ full workloads

def sample_rows(M, n=48):
    rows = np.unique(np.concatenate([np.linspace(0, M - 1, n).astype(np.int64), [0, M - 1, max(M - 7, 0)]]))
    return rows


# Full-size workloads are compared over their whole outputs in
# tests/test_gpu_full.py.


# --------------------------------------------------------- edge cases

def test_usage_example_shape(dev):
    """README Usage: in=4096, out=16384, rank=64, x (8, 4096) -> y (8, 16384)."""
    d = wl.random_inputs(8, 4096, 16384, 64, seed=3)
    g = to_dev(d, dev)
    say("usage example")
    y = Handle(0).forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    assert y.shape == (8, 16384) and y.dtype == torch.bfloat16
    parity.check(parity.to_f64(y), oracle_y(d), False)


def test_leading_dims_flatten(dev):
    d = wl.random_inputs(24, 256, 96, 8, seed=4)
    g = to_dev(d, dev)
    say("leading dims")
    y = Handle(0).forward(g["x"].view(2, 3, 4, 256), g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    torch.cuda.synchronize()
    assert y.shape == (2, 3, 4, 96)
    parity.check(parity.to_f64(y.reshape(24, 96)), oracle_y(d), False)


@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_degenerate_cases(dev, path):
    h = make_handle(dev, path)
    # r = 0: pure scaled residual; no bias
    d = wl.random_inputs(12, 128, 72, 0, seed=5, with_bias=False)
    say("r=0 no bias", path.name)
    parity.check(parity.to_f64(run(h, to_dev(d, dev))), oracle_y(d), False)
    # Q = 0: pure low-rank (the SVDLinearLayer forward)
    d = wl.random_inputs(12, 128, 72, 16, seed=6)
    d["Q"] = torch.zeros_like(d["Q"])
    say("Q=0", path.name)
    parity.check(parity.to_f64(run(h, to_dev(d, dev))), oracle_y(d), False)
    # A = B = 0: pure scaled residual through the rank-r machinery
    d = wl.random_inputs(12, 128, 72, 16, seed=7)
    d["A"], d["B"] = torch.zeros_like(d["A"]), torch.zeros_like(d["B"])
    say("A=B=0", path.name)
    parity.check(parity.to_f64(run(h, to_dev(d, dev))), oracle_y(d), False)
    # scale = 0 and an extreme scale (the tiled path's unfolded order)
    for s in (0.0, 2.0 ** -70, 2.0 ** 70):
        d = wl.random_inputs(12, 128, 72, 16, seed=8)
        d["scale"] = s
        say("scale", s, path.name)
        parity.check(parity.to_f64(run(h, to_dev(d, dev))), oracle_y(d), False)


def test_in_zero_gives_bias(dev):
    say("in=0")
    N = 40
    bias = (torch.arange(N, dtype=torch.float32) / 8).to(torch.bfloat16).to(dev)
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=dev)
    Q = torch.empty((N, 0), dtype=torch.uint8, device=dev)
    A = torch.ones((N, 4), dtype=torch.bfloat16, device=dev)
    B = torch.empty((4, 0), dtype=torch.bfloat16, device=dev)
    y = Handle(0).forward(x, A, B, Q, 1.0, bias)
    torch.cuda.synchronize()
    assert torch.equal(y, bias.expand(5, N))


def test_empty_m_is_a_noop(dev):
    say("M=0")
    d = wl.random_inputs(0, 64, 32, 4, seed=9)
    g = to_dev(d, dev)
    out = torch.full((0, 32), 7.0, dtype=torch.bfloat16, device=dev)
    y = Handle(0).forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=out)
    assert y.shape == (0, 32)


@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_no_stores_outside_y(dev, path):
    """Canary regions around y stay untouched (ragged M and out)."""
    M, K, N, r = 37, 256, 203, 20
    d = wl.random_inputs(M, K, N, r, seed=10)
    g = to_dev(d, dev)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), -77.0, dtype=torch.bfloat16, device=dev)
    y = buf[pad:pad + M * N].view(M, N)
    say("canary", path.name)
    make_handle(dev, path).forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=y)
    torch.cuda.synchronize()
    assert bool((buf[:pad] == -77.0).all()) and bool((buf[pad + M * N:] == -77.0).all())
    parity.check(parity.to_f64(y), oracle_y(d), False)


@pytest.mark.parametrize("path", PATHS, ids=["skinny", "tiled"])
def test_repeat_is_bitwise_deterministic(dev, path):
    d = wl.random_inputs(48, 1024, 1000, 64, seed=11)
    g = to_dev(d, dev)
    h = make_handle(dev, path)
    say("determinism", path.name)
    assert torch.equal(run(h, g), run(h, g))


def test_bad_arguments_return_status(dev):
    d = wl.random_inputs(16, 64, 32, 4, seed=12)
    g = to_dev(d, dev)
    h = Handle(0)
    say("bad args")
    with pytest.raises(LiteLinearError) as e:  # misaligned x (offset by one element)
        xs = torch.zeros(16 * 64 + 1, dtype=torch.bfloat16, device=dev)[1:].view(16, 64)
        h.forward(xs, g["A"], g["B"], g["Q"], g["scale"], g["bias"])
    assert e.value.status == Status.UNSUPPORTED
    with pytest.raises(LiteLinearError) as e:  # y aliases x
        h.forward(g["x"], g["A"], g["B"], g["Q"], g["scale"], g["bias"], out=g["x"].view(-1)[:16 * 32].view(16, 32))
    assert e.value.status == Status.INVALID_ARG
    h.set_option(Option.PATH, int(Path.SKINNY))
    with pytest.raises(LiteLinearError) as e:  # the skinny kernel does not take M > 64
        d2 = to_dev(wl.random_inputs(65, 64, 32, 4, seed=13), dev)
        h.forward(d2["x"], d2["A"], d2["B"], d2["Q"], d2["scale"], d2["bias"])
    assert e.value.status == Status.UNSUPPORTED
    for key, bad in ((Option.PATH, 3), (Option.OUTPUT_F32, 2), (Option.SPLIT_K, -1), (Option.PROFILE, 5),
                     (Option.T_SPLITS, 65), (Option.T_SPLITS, -1), (Option.T_LAUNCH, 3), (Option.T_LAUNCH, -1),
                     (99, 0)):
        with pytest.raises(LiteLinearError) as e:
            h.set_option(key, bad)
        assert e.value.status == Status.INVALID_ARG


def test_profiling_counts_launches(dev):
    d = wl.random_inputs(128, 256, 256, 20, seed=14)   # r % 8 != 0: A is padded first
    g = to_dev(d, dev)
    h = make_handle(dev, Path.TILED)
    h.set_option(Option.PROFILE, 1)
    say("profile")
    for _ in range(3):
        y = run(h, g)
    parity.check(parity.to_f64(y), oracle_y(d), False)
    ms, n = h.kernel_time(Kernel.MAIN)
    assert n == 3 and ms > 0
    ms, n = h.kernel_time(Kernel.PAD_A, reset=True)
    assert n == 3
    assert h.kernel_time(Kernel.PAD_A) == (0.0, 0)
    assert h.kernel_time(Kernel.SKINNY) == (0.0, 0)
