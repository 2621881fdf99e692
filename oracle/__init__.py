"""CPU oracle for the fused LiteLinear forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it, and it imports nothing from them.

It wraps ``litelinear_oracle.c`` (plain C, float64, exact e4m3fn decode by
the closed form of the OCP format) through ctypes.  The forward it computes is
the equation in the introduction of the LiteLinear README (page
"moonmath-ai/LiteLinear"):

    y = (x B^T) A^T + scale * (x dec(Q)^T) + bias

with A [out, r], B [r, in] and Q [out, in] as the README's Features list and
the tt_compressor page's ``SVDLinearLayer`` lay them out.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

_LIB = None


def library(path: str | None = None):
    """Load (building on first use) the oracle's shared library."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _bind(ctypes.CDLL(_build.LIB))
    return _LIB


def _bind(lib):
    lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_decode_e4m3fn.restype = None
    lib.oracle_forward_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_forward_rows.restype = ctypes.c_int
    lib.oracle_forward_rows_q.argtypes = lib.oracle_forward_rows.argtypes + [ctypes.c_int]
    lib.oracle_forward_rows_q.restype = ctypes.c_int
    lib.oracle_e4m3fnuz_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fnuz_to_f64.restype = ctypes.c_double
    lib.oracle_decode_e4m3fnuz.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_decode_e4m3fnuz.restype = None
    lib.oracle_quantize_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.oracle_quantize_rows.restype = None
    lib.oracle_forward_rows_act8.argtypes = lib.oracle_forward_rows.argtypes
    lib.oracle_forward_rows_act8.restype = ctypes.c_int
    lib.oracle_residual.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_residual.restype = None
    lib.oracle_quantize_tensor.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_quantize_tensor.restype = ctypes.c_float
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _bits16(t: torch.Tensor | None) -> np.ndarray | None:
    if t is None:
        return None
    assert t.dtype == torch.bfloat16, t.dtype
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy()).view(np.uint16)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode_e4m3fn(codes, lib=None) -> np.ndarray:
    """e4m3fn codes (any integer array or uint8 tensor) -> float64 values."""
    lib = lib or library()
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.int64).astype(np.uint8))
    out = np.empty(c.shape, np.float64)
    lib.oracle_decode_e4m3fn(_ptr(c), c.size, _ptr(out))
    return out


def decode_e4m3fnuz(codes, lib=None) -> np.ndarray:
    """e4m3fnuz codes (any integer array or uint8 tensor) -> float64 values."""
    lib = lib or library()
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.int64).astype(np.uint8))
    out = np.empty(c.shape, np.float64)
    lib.oracle_decode_e4m3fnuz(_ptr(c), c.size, _ptr(out))
    return out


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def quantize_rows(x: torch.Tensor, lib=None):
    """Activations in e4m3fn with one power-of-two scale per row.

    x bf16 [M, in] -> (codes uint8 [M, in], e int32 [M]) with
    x[m, j] ~ 2^e[m] * dec(codes[m, j]): e[m] is the smallest integer (at
    least -126) with max_j |x[m, j]| <= 448 * 2^e[m], each code the nearest
    e4m3fn value to x[m, j] / 2^e[m] with ties to even.  A row holding a NaN
    or an infinity gets e = 0 and all codes 0x7F (NaN).
    """
    lib = lib or library()
    xb = _bits16(x)
    M, K = xb.shape
    codes = np.empty((M, K), np.uint8)
    exps = np.empty(M, np.int32)
    lib.oracle_quantize_rows(_ptr(xb), M, K, _ptr(codes), _ptr(exps))
    return codes, exps


def residual(W: torch.Tensor, A: torch.Tensor, B: torch.Tensor, lib=None) -> np.ndarray:
    """R = W - A B in float64 (W bf16 [out, in], A bf16 [out, r], B bf16 [r, in])."""
    lib = lib or library()
    out, K = W.shape
    r = A.shape[1]
    assert A.shape == (out, r) and B.shape == (r, K)
    Wb, Ab, Bb = _bits16(W), _bits16(A), _bits16(B)
    R = np.empty((out, K), np.float64)
    lib.oracle_residual(_ptr(Wb), _ptr(Ab), _ptr(Bb), out, K, r, _ptr(R))
    return R


def quantize_tensor(R, lib=None):
    """Per-tensor e4m3fn codes of a float32 array: (codes uint8, scale float).

    scale = amax / 448 in float32 (1 for an all-zero array); each code is the
    e4m3fn value nearest to the float32 quotient R / scale clamped to +-448.
    """
    lib = lib or library()
    Rf = np.ascontiguousarray(np.asarray(R, dtype=np.float32))
    codes = np.empty(Rf.shape, np.uint8)
    s = lib.oracle_quantize_tensor(_ptr(Rf), Rf.size, _ptr(codes))
    return codes, float(np.float32(s))


def gelu_tanh(v) -> np.ndarray:
    """GELU in its tanh approximation, in float64 (Hendrycks and Gimpel,
    "Gaussian Error Linear Units (GELUs)", 2016, section 2):
    0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).  The activation that the
    library's activation option fuses into its epilogue, applied here to the
    oracle's float64 forward."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)))


def gelu_erf(v) -> np.ndarray:
    """The exact GELU in float64 (Hendrycks and Gimpel, "Gaussian Error Linear
    Units (GELUs)", 2016, section 2): v Phi(v) = 0.5 v (1 + erf(v / sqrt(2))),
    Phi the standard normal distribution function (erf from scipy)."""
    from scipy.special import erf

    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def geglu(y_pre) -> np.ndarray:
    """GEGLU of a projection's output (Shazeer, "GLU Variants Improve
    Transformer", 2020): the 2F columns of y_pre are split into a hidden half
    [:, :F] and a gate half [:, F:], and the result is hidden * GELU(gate),
    the exact GELU, in float64 -- the gated feed-forward input that the
    LiteLinear README's integration guide replaces with a LiteLinear
    projection (LTX-style models wrap the first linear in a GEGLU)."""
    y_pre = np.asarray(y_pre, dtype=np.float64)
    F = y_pre.shape[-1] // 2
    assert y_pre.shape[-1] == 2 * F, "GEGLU needs an even number of columns"
    return y_pre[..., :F] * gelu_erf(y_pre[..., F:])


def forward(x: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None,
            Q: torch.Tensor, scale: float, bias: torch.Tensor | None,
            rows=None, threads: int | None = None, want_T: bool = False, lib=None,
            act_fp8: bool = False, q_format: str = "e4m3fn"):
    """float64 forward for all rows of x, or for the row indices in ``rows``.

    x bf16 [M, in]; A bf16 [out, r]; B bf16 [r, in]; Q uint8 e4m3fn codes
    [out, in]; scale a float32 value; bias bf16 [out] or None.  Returns y as
    float64 [len(rows), out], plus T [len(rows), r] when ``want_T``.
    With ``act_fp8`` the residual product reads x quantised by
    ``quantize_rows`` (the fp8-activation mode); T still reads the bf16 x.
    ``q_format`` "e4m3fnuz" decodes Q as e4m3fnuz codes (bf16 activations).
    """
    if q_format not in ("e4m3fn", "e4m3fnuz"):
        raise ValueError(q_format)
    if act_fp8 and q_format != "e4m3fn":
        raise ValueError("the fp8-activation forward takes e4m3fn codes")
    lib = lib or library()
    M, K = x.shape
    N = Q.shape[0]
    r = 0 if A is None else A.shape[1]
    assert Q.shape == (N, K) and Q.dtype == torch.uint8
    if r:
        assert A.shape == (N, r) and B.shape == (r, K)
    xb, Ab, Bb, bb = _bits16(x), _bits16(A) if r else None, _bits16(B) if r else None, _bits16(bias)
    Qb = np.ascontiguousarray(Q.detach().cpu().contiguous().numpy())
    if rows is None:
        ridx = None
        nrows = M
    else:
        ridx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = ridx.size
    y = np.empty((nrows, N), np.float64)
    T = np.empty((nrows, max(r, 1)), np.float64) if want_T else None
    args = (_ptr(xb), _ptr(Ab), _ptr(Bb), _ptr(Qb), ctypes.c_float(scale),
            _ptr(bb), M, K, N, r, _ptr(ridx), nrows, _ptr(y), _ptr(T),
            int(threads or default_threads()))
    if act_fp8:
        rc = lib.oracle_forward_rows_act8(*args)
    else:
        rc = lib.oracle_forward_rows_q(*args, 1 if q_format == "e4m3fnuz" else 0)
    if rc != 0:
        raise ValueError("oracle_forward_rows rejected its arguments")
    if want_T:
        return y, T[:, :r]
    return y
