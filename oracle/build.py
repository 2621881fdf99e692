"""Builds the CPU oracle's shared library with gcc (test infrastructure)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "litelinear_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(out: str = LIB, plant: int = 0, quiet: bool = True) -> str:
    """Compile the oracle; ``plant`` > 0 builds a deliberately wrong variant."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", f"-DORACLE_PLANT={int(plant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False), file=sys.stderr)
