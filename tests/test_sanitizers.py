"""CPU: the oracle and the host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU code is built with a sanitizer).

- tests/sanitize/oracle_check.c runs every exported oracle function on small and ragged
  inputs and on invalid arguments.
- tests/sanitize/host_check.cpp compiles the library's host sources (argument validation,
  the table caches and the host table builders) with host stand-ins for the HIP runtime
  and the kernel launchers. It then drives every entry point and checks the arguments that
  reach the launchers. The library's table caches live until the process ends by design;
  the leak checker is told so (tests/sanitize/lsan_cache.supp) and checks everything else.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, tmp_path):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["LSAN_OPTIONS"] = "suppressions=%s:print_suppressions=0" % os.path.join(ROOT, "tests", "sanitize",
                                                                              "lsan_cache.supp")
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, cwd=tmp_path, env=env)


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    r = subprocess.run(["gcc", "-std=c99", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
                        os.path.join(ROOT, "oracle", "tra_oracle.c"), "-o", exe, "-lm", "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = _run(exe, tmp_path)
    assert r.returncode == 0 and "oracle sanitize ok" in r.stdout, r.stderr[-4000:]


def test_host_library_under_sanitizers(tmp_path):
    inc = "/opt/rocm/include"
    if shutil.which("g++") is None or not os.path.exists(os.path.join(inc, "hip", "hip_runtime.h")):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path / "host_check")
    r = subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I",
                        os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "entropy_adaptive_sparse_amd", "csrc"),
                        os.path.join(ROOT, "tests", "sanitize", "host_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = _run(exe, tmp_path)
    assert r.returncode == 0 and "host sanitize ok" in r.stdout, r.stderr[-4000:]
