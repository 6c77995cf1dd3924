"""Shared helpers for the GPU parity tests (inputs from the seeded generator, the
oracle on the CPU, the HIP path through the C ABI binding)."""
import math
import sys

import numpy as np

from entropy_adaptive_sparse_amd import synth
from entropy_adaptive_sparse_amd import workloads


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def device():
    torch = torch_mod()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def tra():
    import entropy_adaptive_sparse_amd as t
    t.load()  # fail loudly if the HIP library is missing
    return t


def qkv_inputs(wl, heads=None, dtype=None):
    """Natural-order q, k, v for workload wl as CPU torch tensors of the workload dtype."""
    torch = torch_mod()
    q, k, v = synth.qkv(wl.wid, wl.outer, wl.F, wl.H, wl.W, wl.D, wl.t_lo, wl.t_hi, heads=heads)
    dt = dtype or (torch.float32 if wl.dtype == "f32" else torch.bfloat16)
    return tuple(torch.from_numpy(x).to(dt) for x in (q, k, v))


def small_workload(wid, F, H, W, D, dtype, outer=2, bq=128, bk=64, tau=0.05, gamma=0.5, vote=1, t_lo=0.25,
                   t_hi=8.0):
    return workloads.Workload(wid, "test-%dx%dx%d" % (F, H, W), 1, outer, D, dtype, F, H, W, bq, bk, tau, gamma,
                              vote, 8, 8, t_lo, t_hi)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_output(got, ref, dtype):
    """Tolerances: fp32 max-abs <= 1e-4; bf16 relative L2 <= 1e-2 and max-abs <= 3e-2."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if dtype == "f32":
        assert err <= 1e-4, "fp32 max-abs %.3g" % err
        return err, rel_l2(got, ref)
    rl = rel_l2(got, ref)
    assert rl <= 1e-2 and err <= 3e-2, "bf16 rel-L2 %.3g max-abs %.3g" % (rl, err)
    return err, rl


def sample_rows(seed, N, bq, nblocks):
    """Seeded q-blocks -> the query positions (tile-major) they hold, plus the blocks."""
    nqb = -(-N // bq)
    blocks = synth.uniform_ints(seed, nblocks - 1, 0, nqb - 1).tolist() + [nqb - 1]  # always the ragged one
    rows = np.concatenate([np.arange(b * bq, min(N, b * bq + bq)) for b in blocks]).astype(np.int32)
    return np.array(blocks, dtype=np.int32), rows
