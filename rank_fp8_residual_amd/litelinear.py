"""Thin ctypes binding of liblitelinear.so (see include/litelinear.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity and handed over as device pointers with torch's current HIP
stream.  Every step of the forward runs in the library's HIP kernels; there
is no other implementation to fall back to, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import enum
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblitelinear.so")

_lib = None
_lib_lock = threading.Lock()


class Status(enum.IntEnum):
    OK = 0
    INVALID_ARG = 1
    UNSUPPORTED = 2
    HIP = 3
    OOM = 4
    SYNC = 5  # an earlier launch gave up waiting for other work-groups (see device_status)
    SCRATCH = 6  # forward_noalloc: more workspace needed than the fixed scratch holds


class Option(enum.IntEnum):
    PATH = 1
    OUTPUT_F32 = 2
    SPLIT_K = 3
    PROFILE = 4
    T_SPLITS = 5
    ACT_FP8 = 6
    ACTIVATION = 7  # 1 = GELU (tanh approximation) on y, fused into the epilogue
    TEST_WAIT_TIMEOUT = 8  # test hook: n > 0 makes every bounded wait give up after n polls
    Q_FORMAT = 9  # residual codes: 0 e4m3fn, 1 e4m3fnuz
    T_LAUNCH = 10  # tiled path: T by 0 = automatic choice, 1 = in-launch producers, 2 = a launch of its own


class Activation(enum.IntEnum):
    NONE = 0
    GELU_TANH = 1  # GELU (tanh approximation) on every element of y
    GEGLU = 2      # y [M, out/2] = hidden * GELU_erf(gate), halves of the 2F-row projection


class Path(enum.IntEnum):
    AUTO = 0
    SKINNY = 1
    TILED = 2


class Kernel(enum.IntEnum):
    PAD_A = 0
    MAIN = 1
    SKINNY = 2
    QUANT = 3
    CONVERT = 4


EXPORTS = ("litelinear_create", "litelinear_forward", "litelinear_destroy", "litelinear_check_args",
           "litelinear_set_option", "litelinear_kernel_time", "litelinear_status_string",
           "litelinear_version", "litelinear_quantize_rows", "litelinear_quantize_tensor",
           "litelinear_residual_quantize", "litelinear_forward_pair", "litelinear_forward_strided",
           "litelinear_device_status", "litelinear_read_probe", "litelinear_forward_noalloc")


class LiteLinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = Status(status) if status in Status._value2member_map_ else status
        super().__init__(f"{what}: {lib().litelinear_status_string(status).decode()} (status {status})")


def lib(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library; raises ImportError when it has not been built."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"liblitelinear.so not found at {p}; build it with "
                          "`python -m rank_fp8_residual_amd.build`")
    with _lib_lock:
        L = ctypes.CDLL(p)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.litelinear_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int]
        L.litelinear_create.restype = ctypes.c_int
        L.litelinear_destroy.argtypes = [vp]
        L.litelinear_destroy.restype = ctypes.c_int
        L.litelinear_forward.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i64, i64, i64, i64, vp]
        L.litelinear_forward.restype = ctypes.c_int
        L.litelinear_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i64, i64, i64, i64, vp]
        L.litelinear_forward_noalloc.restype = ctypes.c_int
        L.litelinear_forward_strided.argtypes = [vp, vp, i64, vp, vp, vp, ctypes.c_float, vp, vp, i64, i64, i64,
                                                 i64, vp]
        L.litelinear_forward_strided.restype = ctypes.c_int
        L.litelinear_check_args.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int]
        L.litelinear_check_args.restype = ctypes.c_int
        L.litelinear_set_option.argtypes = [vp, ctypes.c_int, i64]
        L.litelinear_set_option.restype = ctypes.c_int
        L.litelinear_kernel_time.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(i64), ctypes.c_int]
        L.litelinear_kernel_time.restype = ctypes.c_int
        L.litelinear_status_string.argtypes = [ctypes.c_int]
        L.litelinear_status_string.restype = ctypes.c_char_p
        L.litelinear_quantize_rows.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.litelinear_quantize_rows.restype = ctypes.c_int
        L.litelinear_quantize_tensor.argtypes = [vp, vp, i64, vp, vp, vp]
        L.litelinear_quantize_tensor.restype = ctypes.c_int
        L.litelinear_residual_quantize.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]
        L.litelinear_residual_quantize.restype = ctypes.c_int
        L.litelinear_forward_pair.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i64, vp, vp,
                                              ctypes.c_float, vp, vp, i64, i64, i64, i64, vp]
        L.litelinear_forward_pair.restype = ctypes.c_int
        L.litelinear_read_probe.argtypes = [vp, vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        L.litelinear_read_probe.restype = ctypes.c_int
        L.litelinear_device_status.argtypes = [vp]
        L.litelinear_device_status.restype = ctypes.c_int
        L.litelinear_version.argtypes = []
        L.litelinear_version.restype = ctypes.c_char_p
        if path is None:
            _lib = L
    return L


def _check(status: int, what: str):
    if status != Status.OK:
        raise LiteLinearError(status, what)


def check_args(x, A, B, Q, bias, y, M, in_features, out_features, r, y_bytes_per_elem=2) -> Status:
    """Host-only argument validation on raw integer addresses (no device use)."""
    return Status(lib().litelinear_check_args(x, A, B, Q, bias, y, M, in_features, out_features, r,
                                              y_bytes_per_elem))


class Handle:
    """Owns one litelinear handle (and its workspace) on one HIP device."""

    def __init__(self, device: int | torch.device | None = None):
        if device is None:
            device = torch.cuda.current_device()
        dev = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
        # always with an index: argument checks compare it with get_device()
        self.device = torch.device("cuda", dev.index if dev.index is not None else torch.cuda.current_device())
        self._h = ctypes.c_void_p()
        _check(lib().litelinear_create(ctypes.byref(self._h), self.device.index or 0), "litelinear_create")
        self.out_f32 = False
        self.activation = Activation.NONE

    def close(self):
        if self._h:
            _check(lib().litelinear_destroy(self._h), "litelinear_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            if self._h:
                lib().litelinear_destroy(self._h)
        except Exception:
            pass

    def set_option(self, key: Option | int, value: int):
        _check(lib().litelinear_set_option(self._h, int(key), int(value)), f"set_option({key})")
        if int(key) == Option.OUTPUT_F32:
            self.out_f32 = bool(value)
        if int(key) == Option.ACTIVATION:
            self.activation = Activation(value)

    def kernel_time(self, kind: Kernel | int, reset: bool = False):
        """(total milliseconds, launches) recorded for one kernel kind."""
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib().litelinear_kernel_time(self._h, int(kind), ctypes.byref(ms), ctypes.byref(n), int(reset)),
               "kernel_time")
        return ms.value, n.value

    def device_status(self) -> Status:
        """SYNC if a bounded wait inside a launch on this handle gave up since
        the last report (that launch's output is undefined), else OK; reads
        the error word without synchronising and clears it."""
        return Status(lib().litelinear_device_status(self._h))

    def read_probe(self, src: torch.Tensor, sink: torch.Tensor, work_groups: int, unroll: int = 8,
                   nontemporal: bool = False, stream: torch.cuda.Stream | None = None):
        """Diagnostic: read all of `src` once (the HBM read ceiling; see
        litelinear_read_probe); `sink` is int32/uint32 with >= work_groups
        elements."""
        _expect(src, "src", src.dtype, self.device, None)
        _expect(sink, "sink", sink.dtype, self.device, None)
        if sink.element_size() != 4 or sink.numel() < work_groups:
            raise ValueError("sink must hold work_groups 32-bit words")
        nbytes = src.numel() * src.element_size()
        _check(lib().litelinear_read_probe(self._h, src.data_ptr(), nbytes, work_groups, unroll, int(nontemporal),
                                           sink.data_ptr(), _stream_ptr(stream, self.device)), "litelinear_read_probe")

    def forward(self, x: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, Q: torch.Tensor,
                scale: float, bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                stream: torch.cuda.Stream | None = None, noalloc: bool = False) -> torch.Tensor:
        """y = (x B^T) A^T + scale * (x dec(Q)^T) + bias on this handle's device.

        x may be a row slice of a wider tensor (last dimension contiguous,
        rows evenly spaced after flattening the leading dimensions, e.g.
        ``big[:, :in]``): it is then read in place with its row stride.
        ``noalloc``: litelinear_forward_noalloc (the workspace from the
        library's fixed per-device scratch; contiguous x; pass ``out`` to
        allocate nothing on this side either)."""
        dev = self.device
        if Q.dtype in (torch.float8_e4m3fn, torch.float8_e4m3fnuz):
            Q = Q.view(torch.uint8)
        _expect(Q, "Q", torch.uint8, dev, 2)
        out_features, in_features = Q.shape
        # the gated epilogue's output has half as many columns as Q has rows
        y_cols = out_features // 2 if self.activation == Activation.GEGLU else out_features
        _expect(x, "x", torch.bfloat16, dev, None, contiguous=False)
        if x.shape[-1] != in_features:
            raise ValueError(f"x has {x.shape[-1]} features, Q has {in_features}")
        lead = x.shape[:-1]
        if x.numel() == 0:  # nothing is read: any strides
            x2, ldx = x.reshape(math.prod(lead), in_features), in_features
        else:
            if in_features > 1 and x.stride(-1) != 1:
                raise ValueError("x's last dimension must be contiguous")
            try:
                x2 = x if x.dim() == 2 else x.view(math.prod(lead), in_features)
            except RuntimeError:
                raise ValueError("x's leading dimensions must flatten to rows of one stride") from None
            ldx = x2.stride(0) if x2.shape[0] > 1 else in_features
        M = x2.shape[0]
        if A is None or B is None:
            if (A is None) != (B is None):
                raise ValueError("A and B must both be given or both be None")
            r = 0
        else:
            _expect(A, "A", torch.bfloat16, dev, 2)
            _expect(B, "B", torch.bfloat16, dev, 2)
            r = A.shape[1]
            if A.shape[0] != out_features or B.shape != (r, in_features):
                raise ValueError(f"A {tuple(A.shape)} / B {tuple(B.shape)} do not match "
                                 f"out={out_features}, in={in_features}")
        if bias is not None:
            _expect(bias, "bias", torch.bfloat16, dev, 1)
            if bias.shape[0] != out_features:
                raise ValueError("bias must have out_features elements")
        ydt = torch.float32 if self.out_f32 else torch.bfloat16
        if out is None:
            out = torch.empty((M, y_cols), dtype=ydt, device=dev)
        else:
            _expect(out, "out", ydt, dev, None)
            if out.numel() != M * y_cols:
                raise ValueError("out has the wrong number of elements")
        s = _stream_ptr(stream, dev)
        if noalloc:
            if ldx != in_features:
                raise ValueError("forward_noalloc takes contiguous rows of x")
            st = lib().litelinear_forward_noalloc(self._h, _ptr(x2), _ptr(A) if r else None, _ptr(B) if r else None,
                                                  _ptr(Q), float(scale), _ptr(bias), _ptr(out), M, in_features,
                                                  out_features, r, s)
        elif ldx == in_features:
            st = lib().litelinear_forward(self._h, _ptr(x2), _ptr(A) if r else None, _ptr(B) if r else None,
                                          _ptr(Q), float(scale), _ptr(bias), _ptr(out), M, in_features,
                                          out_features, r, s)
        else:
            st = lib().litelinear_forward_strided(self._h, _ptr(x2), ldx, _ptr(A) if r else None,
                                                  _ptr(B) if r else None, _ptr(Q), float(scale), _ptr(bias),
                                                  _ptr(out), M, in_features, out_features, r, s)
        if st:
            _check(st, "litelinear_forward")
        return out if out.dim() == 2 and len(lead) == 1 else out.view(*lead, y_cols)

    def forward_pair(self, x: torch.Tensor, B: torch.Tensor | None, first: tuple, second: tuple,
                     out: tuple | None = None, stream: torch.cuda.Stream | None = None):
        """Two outputs sharing x and B (T computed once): `first` and `second`
        are (A, Q, scale, bias) tuples; returns (y1, y2)."""
        dev = self.device
        _expect(x, "x", torch.bfloat16, dev, None)
        in_features = x.shape[-1]
        lead = x.shape[:-1]
        x2 = x.reshape(math.prod(lead), in_features)
        if not x2.is_contiguous():
            raise ValueError("x must be contiguous")
        M = x2.shape[0]
        r = 0 if B is None else B.shape[0]
        if B is not None:
            _expect(B, "B", torch.bfloat16, dev, 2)
            if B.shape[1] != in_features:
                raise ValueError("B does not match x")
        sets = []
        for name, (A, Q, scale, bias) in (("first", first), ("second", second)):
            if Q.dtype == torch.float8_e4m3fn:
                Q = Q.view(torch.uint8)
            _expect(Q, f"{name} Q", torch.uint8, dev, 2)
            n_out = Q.shape[0]
            if Q.shape[1] != in_features:
                raise ValueError(f"{name} Q does not match x")
            if (A is None) != (B is None):
                raise ValueError("A must be given exactly when B is")
            if A is not None:
                _expect(A, f"{name} A", torch.bfloat16, dev, 2)
                if A.shape != (n_out, r):
                    raise ValueError(f"{name} A must be [{n_out}, {r}]")
            if bias is not None:
                _expect(bias, f"{name} bias", torch.bfloat16, dev, 1)
                if bias.shape[0] != n_out:
                    raise ValueError(f"{name} bias must have {n_out} elements")
            sets.append((A, Q, float(scale), bias, n_out))
        ydt = torch.float32 if self.out_f32 else torch.bfloat16
        ys = []
        for i, (_, _, _, _, n_out) in enumerate(sets):
            y = out[i] if out is not None else torch.empty((M, n_out), dtype=ydt, device=dev)
            _expect(y, "out", ydt, dev, None)
            if y.numel() != M * n_out:
                raise ValueError("out has the wrong number of elements")
            ys.append(y)
        s = _stream_ptr(stream, dev)
        ptr = lambda t: None if t is None or t.numel() == 0 else t.data_ptr()
        (A1, Q1, s1, b1, n1), (A2, Q2, s2, b2, n2) = sets
        st = lib().litelinear_forward_pair(self._h, ptr(x2), ptr(B) if r else None, ptr(A1) if r else None, ptr(Q1),
                                           ctypes.c_float(s1), ptr(b1), ptr(ys[0]), n1,
                                           ptr(A2) if r else None, ptr(Q2), ctypes.c_float(s2), ptr(b2), ptr(ys[1]),
                                           n2, M, in_features, r, s)
        _check(st, "litelinear_forward_pair")
        return ys[0].view(*lead, n1), ys[1].view(*lead, n2)

    def quantize_rows(self, x: torch.Tensor, codes: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
        """x bf16 [M, in] -> (e4m3fn codes uint8 [M, in], row scales float32 [M]),
        x[m, j] ~ scales[m] * dec(codes[m, j]) (see litelinear_quantize_rows)."""
        dev = self.device
        _expect(x, "x", torch.bfloat16, dev, 2)
        M, K = x.shape
        if codes is None:
            codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
        else:
            _expect(codes, "codes", torch.uint8, dev, 2)
            if codes.shape != (M, K):
                raise ValueError("codes must have x's shape")
        if scales is None:
            scales = torch.empty((M,), dtype=torch.float32, device=dev)
        else:
            _expect(scales, "scales", torch.float32, dev, 1)
            if scales.shape[0] != M:
                raise ValueError("scales must have one element per row")
        s = _stream_ptr(stream, dev)
        ptr = lambda t: None if t.numel() == 0 else t.data_ptr()
        _check(lib().litelinear_quantize_rows(self._h, ptr(x), M, K, ptr(codes), ptr(scales), s),
               "litelinear_quantize_rows")
        return codes, scales

    def quantize_tensor(self, R: torch.Tensor, stream: torch.cuda.Stream | None = None):
        """float32 R -> (e4m3fn codes uint8 of R's shape, scale float32 [1] on
        the device), R ~ scale * dec(codes) (see litelinear_quantize_tensor)."""
        dev = self.device
        _expect(R, "R", torch.float32, dev, None)
        codes = torch.empty(R.shape, dtype=torch.uint8, device=dev)
        scale = torch.empty((1,), dtype=torch.float32, device=dev)
        s = _stream_ptr(stream, dev)
        ptr = lambda t: None if t.numel() == 0 else t.data_ptr()
        _check(lib().litelinear_quantize_tensor(self._h, ptr(R), R.numel(), ptr(codes), scale.data_ptr(), s),
               "litelinear_quantize_tensor")
        return codes, scale

    def residual_quantize(self, W: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None,
                          stream: torch.cuda.Stream | None = None):
        """e4m3fn codes and per-tensor scale of R = W - A B (the forward's Q and
        scale for the pair A, B; see litelinear_residual_quantize)."""
        dev = self.device
        _expect(W, "W", torch.bfloat16, dev, 2)
        out_features, in_features = W.shape
        if A is None or B is None:
            if (A is None) != (B is None):
                raise ValueError("A and B must both be given or both be None")
            r = 0
        else:
            _expect(A, "A", torch.bfloat16, dev, 2)
            _expect(B, "B", torch.bfloat16, dev, 2)
            r = A.shape[1]
            if A.shape[0] != out_features or B.shape != (r, in_features):
                raise ValueError("A / B do not match W")
        codes = torch.empty((out_features, in_features), dtype=torch.uint8, device=dev)
        scale = torch.empty((1,), dtype=torch.float32, device=dev)
        s = _stream_ptr(stream, dev)
        ptr = lambda t: None if t is None or t.numel() == 0 else t.data_ptr()
        _check(lib().litelinear_residual_quantize(self._h, ptr(W), ptr(A) if r else None, ptr(B) if r else None,
                                                  out_features, in_features, r, ptr(codes), scale.data_ptr(), s),
               "litelinear_residual_quantize")
        return codes, scale


def _ptr(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, dev: torch.device):
    """The HIP stream to enqueue on: the given one, else torch's current one."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _expect(t, name, dtype, dev, ndim, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.get_device() != dev.index:
        raise ValueError(f"{name} is on {t.device}, the handle on {dev}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_default_handles: dict[int, Handle] = {}


def default_handle(device: int | None = None) -> Handle:
    idx = torch.cuda.current_device() if device is None else device
    h = _default_handles.get(idx)
    if h is None:
        h = _default_handles[idx] = Handle(idx)
    return h


def forward(x, A, B, Q, scale, bias=None, out=None):
    """Functional form on the default handle of x's device."""
    return default_handle(x.device.index).forward(x, A, B, Q, scale, bias, out)
