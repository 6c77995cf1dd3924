"""GPU: the C ABI from a plain C99 program (tests/c_abi_check.c: no Python, no torch).
It runs the permutation round trip, dense attention + entropy, a keep-everything mask, and
block-sparse attention over it, which must equal the dense output bit for bit ("Token
Radius Attention for Efficient Video Generation", section 2, TRA pipeline steps 1-3). It
also checks that an unsupported head size is refused."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_caller():
    assert os.path.exists(EXE), "tests/c_abi_check is built by `python -m entropy_adaptive_sparse_amd.build`"
    say("plain C caller of libtra.so")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stderr
