"""Builds libtra.so (HIP, gfx950) in-tree with hipcc.

    python -m entropy_adaptive_sparse_amd.build

Every source compiles to an object of its own (in parallel), then one shared
library is linked next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtra.so")
SOURCES = ["tra_api.cpp", "mask_sizes.cpp", "permute.hip", "mask.hip", "attention.hip", "schedule.hip", "mask1d.hip"]
ARCH = os.environ.get("TRA_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in r.stderr.splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build_c_check(verbose: bool = False) -> str:
    """The plain-C caller of the ABI used by the GPU tests (tests/c_abi_check.c), linked
    against the in-tree libtra.so and the ROCm HIP runtime."""
    src = os.path.join(ROOT, "tests", "c_abi_check.c")
    exe = os.path.join(ROOT, "tests", "c_abi_check")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), src, "-o", exe, "-L", HERE, "-ltra", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../entropy_adaptive_sparse_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("c_abi_check build failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    if verbose:
        print("built", exe)
    return exe


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_c_check(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
