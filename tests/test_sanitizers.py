"""Host sanitizer build: the oracle and the C ABI's host-only argument
checks compiled with gcc's address and undefined-behaviour sanitizers and
run by a small driver (tests/sanitize/sanitize_driver.c) over every decode,
the oracle's forwards, quantisers and residual, and valid, edge and refused
argument sets.  No GPU; no HIP code is built with a sanitizer."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no host compiler")
def test_oracle_and_host_checks_under_asan_ubsan(tmp_path):
    objs = []

    def cc(cmd, out):
        res = subprocess.run(cmd + ["-o", str(out)], capture_output=True, text=True, cwd=ROOT)
        assert res.returncode == 0, res.stderr[-3000:]
        objs.append(str(out))

    cc(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-c",
        os.path.join(ROOT, "oracle", "litelinear_oracle.c")], tmp_path / "oracle.o")
    cc(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "tests", "sanitize", "sanitize_driver.c")],
       tmp_path / "driver.o")
    cc(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}",
        f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'rank_fp8_residual_amd', 'csrc')}", "-c",
        os.path.join(ROOT, "rank_fp8_residual_amd", "csrc", "check.cpp")], tmp_path / "check.o")
    exe = tmp_path / "sanitize_driver"
    res = subprocess.run(["g++", "-fsanitize=address,undefined", "-fopenmp", *objs, "-o", str(exe), "-lm"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "all checks passed" in run.stdout
    assert "runtime error" not in report and "AddressSanitizer" not in report and "LeakSanitizer" not in report
