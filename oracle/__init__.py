"""Plain fp64 CPU oracle for the Token Radius Attention (TRA) hot path.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU-baseline
leg of ``bench.py`` may import this module; the product package never does,
and this module imports nothing from the product package.

The arithmetic lives in ``tra_oracle.c`` (plain C, fp64, pthreads); this file
only marshals numpy arrays into it.  Each wrapped function names the passage
of "Token Radius Attention for Efficient Video Generation" (gist.science
summary, section 2: Insight I, Insight II, the TRA pipeline) that it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tra_oracle.c")
# TRA_ORACLE_LIB names another build of tra_oracle.c to load (the planted-mistake tests load
# deliberately broken copies this way, in a process of their own)
_LIB = os.environ.get("TRA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, strict fp64: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
               "-pthread", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
            lib.orc_tile_major_order.argtypes = [i32, i32, i32, i32, i32, P]
            lib.orc_attention.argtypes = [P, P, P, i32, i32, f64, P, i32, P, i32, i32, P, P, P, i32]
            lib.orc_token_budget.argtypes = [f64, f64]
            lib.orc_token_budget.restype = f64
            lib.orc_frame_norm.argtypes = [i32, f64, P]
            lib.orc_base_radius.argtypes = [f64, f64, f64]
            lib.orc_base_radius.restype = f64
            lib.orc_lambda_table.argtypes = [i32, f32, f32, P]
            lib.orc_log_table.argtypes = [i32, P]
            lib.orc_member_row.argtypes = [P, i32, i32, i32, f32, f32, i32, i32, i32, P]
            lib.orc_count_naive_disagreements.argtypes = [P, i32, i32, i32, f32, f32, i32, i32]
            lib.orc_count_naive_disagreements.restype = i64
            lib.orc_block_mask.argtypes = [P, i32, i32, i32, f32, f32, i32, i32, i32, i32, i32, P, i32,
                                           P, P, i32]
            lib.orc_window_mu.argtypes = [f32]
            lib.orc_window_mu.restype = f64
            lib.orc_member_row_1d.argtypes = [P, i32, i32, i32, f32, i32, i32, i32, P]
            lib.orc_count_naive_disagreements_1d.argtypes = [P, i32, i32, i32, f32, i32, i32]
            lib.orc_count_naive_disagreements_1d.restype = i64
            lib.orc_block_mask_1d.argtypes = [P, i32, i32, i32, f32, i32, i32, i32, i32, i32, P, i32, P, P, i32]
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


# --------------------------------------------------------------------------------------------
# tile-major order (pipeline step 3, tile-major layout)
# --------------------------------------------------------------------------------------------
def tile_major_order(F: int, H: int, W: int, th: int = 8, tw: int = 8) -> np.ndarray:
    """perm[p] = natural index (f*H+h)*W+w of the token at tile-major position p (enumerated)."""
    perm = np.empty(F * H * W, dtype=np.int64)
    _check(_load().orc_tile_major_order(F, H, W, th, tw, _ptr(perm)), "tile_major_order")
    return perm


def permute(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """y[p] = x[perm[p]] along axis -2 (rows), pure indexing."""
    return np.ascontiguousarray(x[..., perm, :])


def unpermute(y: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x[perm[p]] = y[p] along axis -2."""
    x = np.empty_like(y)
    x[..., perm, :] = y
    return x


# --------------------------------------------------------------------------------------------
# attention + entropy (section 1; pipeline step 1; Insight I)
# --------------------------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None, rows=None,
              block_mask: np.ndarray | None = None, bq: int = 0, bk: int = 0, nthreads: int | None = None):
    """One head: q, k, v [N][D] (upcast to fp64).  Returns (o [R][D], entropy [R], lse [R]) for the
    requested rows (default: all).  With block_mask [nqb][nkb], row i sees only the tokens of the
    retained k-blocks of its q-block (positions taken in the order the arrays are given)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    N, D = q.shape
    assert k.shape == (N, D) and v.shape == (N, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(N, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    R = rows.shape[0]
    o = np.empty((R, D), dtype=np.float64)
    ent = np.empty(R, dtype=np.float64)
    lse = np.empty(R, dtype=np.float64)
    mptr = None
    if block_mask is not None:
        block_mask = np.ascontiguousarray(block_mask, dtype=np.uint8)
        assert block_mask.shape == ((N + bq - 1) // bq, (N + bk - 1) // bk)
        mptr = _ptr(block_mask)
    rc = _load().orc_attention(_ptr(q), _ptr(k), _ptr(v), N, D, float(scale), _ptr(rows), R, mptr,
                               int(bq), int(bk), _ptr(o), _ptr(ent), _ptr(lse),
                               nthreads or default_threads())
    _check(rc, "attention")
    return o, ent, lse


# --------------------------------------------------------------------------------------------
# entropy -> budget -> radius (Insight I formula; Insight II radius and phi(delta))
# --------------------------------------------------------------------------------------------
def token_budget(H: float, tau: float) -> float:
    """K = tau * exp(H) tokens (the budget fraction times N)."""
    return _load().orc_token_budget(float(H), float(tau))


def frame_norm(F: int, gamma: float) -> np.ndarray:
    S = np.empty(F, dtype=np.float64)
    _check(_load().orc_frame_norm(F, float(gamma), _ptr(S)), "frame_norm")
    return S


def base_radius(H: float, tau: float, S_f: float) -> float:
    return _load().orc_base_radius(float(H), float(tau), float(S_f))


def lambda_table(F: int, tau: float, gamma: float) -> np.ndarray:
    lam = np.empty((F, F), dtype=np.float64)
    _check(_load().orc_lambda_table(F, float(tau), float(gamma), _ptr(lam)), "lambda_table")
    return lam


def log_table(tmax: int) -> np.ndarray:
    t = np.empty(tmax + 1, dtype=np.float64)
    _check(_load().orc_log_table(tmax, _ptr(t)), "log_table")
    return t


def member_row(ent: np.ndarray, F, H, W, tau, gamma, i, th=8, tw=8) -> np.ndarray:
    """Support of the query at tile-major position i: uint8[N] over tile-major key positions."""
    ent = np.ascontiguousarray(ent, dtype=np.float32)
    out = np.empty(F * H * W, dtype=np.uint8)
    _check(_load().orc_member_row(_ptr(ent), F, H, W, float(tau), float(gamma), th, tw, int(i), _ptr(out)),
           "member_row")
    return out


def naive_disagreements(ent: np.ndarray, F, H, W, tau, gamma, th=8, tw=8) -> int:
    ent = np.ascontiguousarray(ent, dtype=np.float32)
    n = _load().orc_count_naive_disagreements(_ptr(ent), F, H, W, float(tau), float(gamma), th, tw)
    if n < 0:
        raise ValueError("oracle naive_disagreements rejected its arguments")
    return int(n)


# --------------------------------------------------------------------------------------------
# token-level disks -> block-sparse mask (pipeline step 3: distance, radius compare, voting)
# --------------------------------------------------------------------------------------------
def block_mask(ent: np.ndarray, F, H, W, tau, gamma, bq, bk, vote_threshold=1, th=8, tw=8,
               qblocks=None, nthreads: int | None = None):
    """Mask rows for the selected q-blocks of one head.  ent: fp32 entropies in tile-major order.
    Returns (mask uint8 [S][nkb], votes int32 [S][nkb])."""
    ent = np.ascontiguousarray(ent, dtype=np.float32)
    N = F * H * W
    assert ent.shape == (N,)
    nqb, nkb = (N + bq - 1) // bq, (N + bk - 1) // bk
    qblocks = np.arange(nqb, dtype=np.int32) if qblocks is None else np.ascontiguousarray(qblocks, np.int32)
    S = qblocks.shape[0]
    mask = np.zeros((S, nkb), dtype=np.uint8)
    votes = np.zeros((S, nkb), dtype=np.int32)
    rc = _load().orc_block_mask(_ptr(ent), F, H, W, float(tau), float(gamma), bq, bk, int(vote_threshold),
                                th, tw, _ptr(qblocks), S, _ptr(mask), _ptr(votes),
                                nthreads or default_threads())
    _check(rc, "block_mask")
    return mask, votes


def mask_to_lists(mask: np.ndarray):
    """(kv_count [S], list of ascending retained k-block indices per row)."""
    counts = mask.sum(axis=1).astype(np.int32)
    lists = [np.nonzero(row)[0].astype(np.int32) for row in mask]
    return counts, lists


# --------------------------------------------------------------------------------------------
# 1D-distance variant (section 4, ablation study: the radius mask replaced by a 1D distance):
# the budget tau * exp(H_i) spent on a window of the natural raster sequence centred on the
# query, 2 |n_i - n_j| <= K_i
# --------------------------------------------------------------------------------------------
def window_mu(tau: float) -> float:
    """mu = ln tau - ln 2 (fp64): key j is in query i's window iff d = 0 or ln d <= H_i + mu."""
    return _load().orc_window_mu(float(tau))


def member_row_1d(ent: np.ndarray, F, H, W, tau, i, th=8, tw=8) -> np.ndarray:
    """Window support of the query at tile-major position i: uint8[N] over tile-major key positions."""
    ent = np.ascontiguousarray(ent, dtype=np.float32)
    out = np.empty(F * H * W, dtype=np.uint8)
    _check(_load().orc_member_row_1d(_ptr(ent), F, H, W, float(tau), th, tw, int(i), _ptr(out)), "member_row_1d")
    return out


def naive_disagreements_1d(ent: np.ndarray, F, H, W, tau, th=8, tw=8) -> int:
    ent = np.ascontiguousarray(ent, dtype=np.float32)
    n = _load().orc_count_naive_disagreements_1d(_ptr(ent), F, H, W, float(tau), th, tw)
    if n < 0:
        raise ValueError("oracle naive_disagreements_1d rejected its arguments")
    return int(n)


def block_mask_1d(ent: np.ndarray, F, H, W, tau, bq, bk, vote_threshold=1, th=8, tw=8, qblocks=None,
                  nthreads: int | None = None):
    """Mask rows of the 1D window support for the selected q-blocks of one head (tile-major
    entropies).  Returns (mask uint8 [S][nkb], votes int32 [S][nkb])."""
    ent = np.ascontiguousarray(ent, dtype=np.float32)
    N = F * H * W
    assert ent.shape == (N,)
    nqb, nkb = (N + bq - 1) // bq, (N + bk - 1) // bk
    qblocks = np.arange(nqb, dtype=np.int32) if qblocks is None else np.ascontiguousarray(qblocks, np.int32)
    S = qblocks.shape[0]
    mask = np.zeros((S, nkb), dtype=np.uint8)
    votes = np.zeros((S, nkb), dtype=np.int32)
    rc = _load().orc_block_mask_1d(_ptr(ent), F, H, W, float(tau), bq, bk, int(vote_threshold), th, tw,
                                   _ptr(qblocks), S, _ptr(mask), _ptr(votes), nthreads or default_threads())
    _check(rc, "block_mask_1d")
    return mask, votes
