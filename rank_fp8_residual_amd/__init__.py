"""Fused LiteLinear forward for AMD Instinct MI355X (gfx950).

    y = (x B^T) A^T + scale * (x dec(Q)^T) + bias

(LiteLinear README, page "moonmath-ai/LiteLinear", equation in the
introduction.)  The work runs in the HIP kernels of ``liblitelinear.so``,
reached through the C ABI in ``include/litelinear.h``; ``litelinear`` is the
ctypes binding and ``workloads`` draws the seeded synthetic inputs.
"""
from .litelinear import (Activation, Handle, Kernel, LiteLinearError, Option, Path, Status, check_args,
                         default_handle, forward, lib)

__all__ = ["Activation", "Handle", "Kernel", "LiteLinearError", "Option", "Path", "Status", "check_args",
           "default_handle", "forward", "lib"]
