"""Builds liblitelinear.so (the HIP kernels and the C ABI) for gfx950 in-tree.

    python -m rank_fp8_residual_amd.build        # or build() from Python

Every source is compiled with hipcc for gfx950 only; packed float32 VALU ops
are disabled (-packed-fp32-ops).  The library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liblitelinear.so")
ARCH = "gfx950"
SOURCES = ["tiled.hip", "skinny.hip", "quant.hip", "convert.hip", "probe.hip", "noalloc.hip", "check.cpp", "api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-command-line-argument"]


# Per-file flags.  skinny.hip: no wave-level rewriting of atomics.  The
# all-of-K kernel takes a ticket with one lane's atomic at its start and
# reads the result many stages later; rewritten for a whole wave, the atomic's
# result is needed at once, and the wave would wait for it there.
EXTRA_FLAGS = {"skinny.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="litelinear_build_") as td:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(td, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc, *COMMON, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        errors = []
        for src, p in procs:
            msg, _ = p.communicate()
            text = msg.decode(errors="replace")
            if p.returncode != 0:
                errors.append(f"--- {src} ---\n{text}")
            elif verbose and text.strip():
                print(text, file=sys.stderr)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
