"""Host-side tests of the C ABI: the library loads, exports every function the
header declares, and its host-only argument checks return the documented
status codes.  Nothing here runs on a GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import rank_fp8_residual_amd as ll
from rank_fp8_residual_amd import litelinear as bind

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "litelinear.h")

OK, INV, UNS = ll.Status.OK, ll.Status.INVALID_ARG, ll.Status.UNSUPPORTED


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(litelinear_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 16, names
    lib = ctypes.CDLL(bind.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bind.EXPORTS)


def test_version_and_status_strings():
    L = ll.lib()
    assert re.fullmatch(rb"\d+\.\d+\.\d+", L.litelinear_version())
    for s in ll.Status:
        assert L.litelinear_status_string(int(s))
    assert L.litelinear_status_string(99) == b"unknown status"


A16 = 1 << 20  # fake, 16-byte aligned addresses: check_args never dereferences


def args(**kw):
    base = dict(x=A16, A=2 * A16, B=3 * A16, Q=4 * A16, bias=5 * A16, y=64 * A16,
                M=4, in_features=32, out_features=8, r=2, y_bytes_per_elem=2)
    base.update(kw)
    return base


def chk(**kw):
    a = args(**kw)
    return ll.check_args(a["x"], a["A"], a["B"], a["Q"], a["bias"], a["y"], a["M"], a["in_features"],
                         a["out_features"], a["r"], a["y_bytes_per_elem"])


@pytest.mark.parametrize("kw,expect", [
    ({}, OK),
    ({"M": 0, "y": 0, "x": 0}, OK),              # nothing to compute
    ({"out_features": 0, "y": 0}, OK),
    ({"M": -1}, INV), ({"in_features": -16}, INV), ({"out_features": -1}, INV), ({"r": -1}, INV),
    ({"y": 0}, INV), ({"x": 0}, INV), ({"Q": 0}, INV),
    ({"A": 0}, INV), ({"B": 0}, INV),
    ({"r": 0, "A": 0, "B": 0}, OK),              # no low-rank pair
    ({"bias": 0}, OK),                           # no bias
    ({"in_features": 0, "x": 0, "Q": 0, "B": 0}, OK),  # y = bias
    ({"in_features": 24}, UNS),                  # in % 16 != 0
    ({"x": A16 + 8}, UNS), ({"Q": 4 * A16 + 4}, UNS), ({"B": 3 * A16 + 2}, UNS),
    ({"A": 2 * A16 + 1}, UNS), ({"bias": 5 * A16 + 1}, UNS),
    ({"y": 64 * A16 + 1}, UNS), ({"y": 64 * A16 + 2, "y_bytes_per_elem": 4}, UNS),
    ({"y_bytes_per_elem": 3}, INV),
    ({"y": A16}, INV),                            # y overlaps x
    ({"y": A16 + 64}, INV),                       # partial overlap with x (x is 256 B)
    ({"y": 4 * A16 - 32}, INV),                   # y (64 B) runs into Q
    ({"y": 5 * A16}, INV),                        # y overlaps bias
    ({"M": 1 << 41}, INV),                        # absurd size
])
def test_check_args_status(kw, expect):
    assert chk(**kw) == expect


def test_null_handle_calls_fail_cleanly():
    L = ll.lib()
    assert L.litelinear_set_option(None, 1, 0) == INV
    assert L.litelinear_kernel_time(None, 0, None, None, 0) == INV
    assert L.litelinear_destroy(None) == OK
    assert L.litelinear_create(None, 0) == INV
    assert L.litelinear_forward(None, None, None, None, None, ctypes.c_float(1.0), None, None,
                                1, 16, 16, 0, None) == INV
    assert L.litelinear_quantize_rows(None, None, 1, 16, None, None, None) == INV
    assert L.litelinear_device_status(None) == INV


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(ImportError):
        bind.lib(str(tmp_path / "missing.so"))


def test_no_oracle_in_product_path():
    """The HIP library and its binding never reference the oracle."""
    pkg = os.path.join(ROOT, "rank_fp8_residual_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "litelinear_oracle" not in text, f
    so = open(bind.LIB_PATH, "rb").read()
    assert b"oracle_" not in so
