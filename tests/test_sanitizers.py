"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with gcc / g++ (-fsanitize=address,undefined, every
report fatal) and run:
  * tests/sanitize/oracle_check.c with oracle/ptpc_oracle.c: every oracle
    function on small odd-shaped inputs with wider pitches;
  * tests/sanitize/abi_fuzz.cpp with the library's host sources
    (scaled_gemm_amd/csrc/ptpc_api.cpp, plan.cpp) and stub launchers: every
    C-ABI entry point over a grid of extents, pitches and pointers including
    negative, misaligned, boundary and extreme values; the stubs check the
    preconditions the real kernel launchers rely on.
No GPU code is built here (the device kernels are not host code).
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
SRC = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "scaled_gemm_amd", "csrc")


def run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)} -> {r.returncode}\n{r.stdout[-4000:]}"
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
         os.path.join(SRC, "oracle_check.c"), os.path.join(ROOT, "oracle", "ptpc_oracle.c"),
         "-lm", "-o", exe])
    out = run([exe], env=dict(ENV, OMP_NUM_THREADS="4"))
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_abi_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_fuzz")
    run(["g++", "-std=c++20", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         os.path.join(SRC, "abi_fuzz.cpp"), os.path.join(CSRC, "ptpc_api.cpp"),
         os.path.join(CSRC, "plan.cpp"), "-o", exe])
    out = run([exe], env=ENV, timeout=600)
    assert " 0 failures" in out, out
