"""The host code under the sanitizers, on the CPU.

- The C ABI's host side (csrc/fp4kv_api.cpp, csrc/fp4kv_int_api.cpp) built
  with g++ under AddressSanitizer + UndefinedBehaviorSanitizer, linked against
  tests/sanitize/launch_stubs.cpp instead of the kernels (the stubs check the
  launch invariants: pointers, sizes, and that the chunk cut tiles the span),
  and driven through every entry point of include/fp4kv.h and
  include/fp4kv_int.h with valid and invalid arguments
  (tests/sanitize/host_api_driver.cpp).
- The C oracle (oracle/fp4kv_oracle.c) under AddressSanitizer +
  UndefinedBehaviorSanitizer, and under ThreadSanitizer (its batch functions
  run on several threads), driven through every function it exports
  (tests/sanitize/oracle_driver.c).

Any sanitizer report aborts the program (no recovery), so a pass means no
report.  Only host compilers are used; no GPU code is built with a
sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_quantised_kv_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIP_INCLUDE = "/opt/rocm/include"
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TSAN_OPTIONS="halt_on_error=1")
ASAN_UBSAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _build_and_run(cmd, exe):
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


def test_host_library_asan_ubsan(tmp_path):
    _need("g++")
    if not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "host_api_driver")
    cmd = (["g++", "-std=c++17"] + ASAN_UBSAN +
           ["-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "fp4kv_api.cpp"), os.path.join(CSRC, "fp4kv_int_api.cpp"),
            os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "host_api_driver.cpp"), "-o", exe])
    out = _build_and_run(cmd, exe)
    assert int(out.split()[1]) > 50                      # launches reached the stubs


def test_oracle_asan_ubsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    cmd = (["gcc", "-std=c11", "-D_GNU_SOURCE", "-pthread"] + ASAN_UBSAN +
           [os.path.join(ROOT, "oracle", "fp4kv_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    _build_and_run(cmd, exe)


def test_oracle_tsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver_tsan")
    cmd = ["gcc", "-std=c11", "-D_GNU_SOURCE", "-pthread", "-O1", "-g", "-fsanitize=thread",
           os.path.join(ROOT, "oracle", "fp4kv_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe]
    _build_and_run(cmd, exe)
