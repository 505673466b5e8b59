"""Sanitizer builds of the host-side C and C++ (no GPU): the fp64 oracle
(oracle/oracle.c) and the library's host code -- the C-ABI argument validation
and planning (csrc/api.cpp) and the page allocator (csrc/pager.cpp) -- compiled
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code
only; nothing here is built for the GPU) and driven by tests/native/*: every
branch of the oracle on small cases, every entry point with invalid arguments,
the validate-only stage on 2000 random shapes and random allocator sequences
with their invariants.  A memory error, a leak or undefined behaviour aborts
the driver, and the test fails."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-O1", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "san_oracle")
    run(["gcc", "-std=c99", "-fopenmp"] + SAN + [os.path.join(ROOT, "oracle", "oracle.c"),
                                                os.path.join(NATIVE, "sanitize_oracle.c"), "-o", exe, "-lm"])
    res = run([exe], env=ENV, timeout=300)
    assert "ok" in res.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "san_host")
    csrc = os.path.join(ROOT, "paged_mla_decode_02_amd", "csrc")
    run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
         "-I", csrc, "-w"] + SAN + [os.path.join(csrc, "api.cpp"), os.path.join(csrc, "pager.cpp"),
                                   os.path.join(NATIVE, "sanitize_host.cpp"), "-o", exe])
    res = run([exe], env=ENV, timeout=300)
    assert "ok" in res.stdout
