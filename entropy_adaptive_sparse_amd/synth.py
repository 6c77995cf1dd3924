"""Seeded synthetic inputs shaped like video-DiT attention activations.

This module only draws random numbers: it holds none of the method's arithmetic,
and both the HIP path's tests/benchmark and the CPU oracle's tests take their
inputs from it.  numpy only (no torch, no HIP).

Recipe (per (batch, head) pair, natural raster token order (f*H + h)*W + w):
  * RNG: numpy Generator(PCG64); root seed ``20260804 + config_id``; one child
    stream per (batch, head) from ``SeedSequence(root).spawn(outer)``.  Each
    child draws, in this order: noise_k, noise_q, noise_v [N][D] ~ N(0, 1)
    float32, then log-temperatures [N] ~ U(ln t_lo, ln t_hi).
  * A smooth 3D sinusoidal positional component pe(f, h, w) in R^D: channel
    pair c in [0, D/2) drives axis a = c mod 3 (f, h or w) at index m = c div 3;
    with M_a pairs on that axis and axis length L_a, the period is
    P = 4 * L_a ** (m / max(M_a - 1, 1)) tokens; pe[2c] = sin(2 pi x_a / P),
    pe[2c+1] = cos(2 pi x_a / P); amplitude alpha = 0.5.
  * q_i = t_i * (noise_q_i + alpha pe_i), k_j = noise_k_j + alpha pe_j,
    v_j = noise_v_j.  The per-query temperature t_i spreads the attention
    entropies over orders of magnitude, as the pages describe for real heads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT_SEED = 20260804
ALPHA = 0.5


def positional(F: int, H: int, W: int, D: int, alpha: float = ALPHA) -> np.ndarray:
    """pe [N][D] float32 in natural raster order."""
    npair = D // 2
    axes = [c % 3 for c in range(npair)]
    counts = [axes.count(a) for a in range(3)]
    lens = (F, H, W)
    f, h, w = np.meshgrid(np.arange(F), np.arange(H), np.arange(W), indexing="ij")
    coords = [f.reshape(-1).astype(np.float64), h.reshape(-1).astype(np.float64), w.reshape(-1).astype(np.float64)]
    pe = np.empty((F * H * W, D), dtype=np.float64)
    for c in range(npair):
        a = axes[c]
        m = c // 3
        period = 4.0 * float(lens[a]) ** (m / max(counts[a] - 1, 1))
        ang = 2.0 * np.pi * coords[a] / period
        pe[:, 2 * c] = np.sin(ang)
        pe[:, 2 * c + 1] = np.cos(ang)
    return (alpha * pe).astype(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def qkv(config_id: int, outer: int, F: int, H: int, W: int, D: int, t_lo: float = 0.25, t_hi: float = 8.0,
        heads=None):
    """Natural-order float32 q, k, v [outer][N][D] (or only the listed heads, same streams)."""
    N = F * H * W
    children = np.random.SeedSequence(ROOT_SEED + config_id).spawn(outer)
    heads = list(range(outer)) if heads is None else list(heads)
    pe = positional(F, H, W, D)
    q = np.empty((len(heads), N, D), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def one(slot_head):
        slot, head = slot_head
        g = np.random.Generator(np.random.PCG64(children[head]))
        g.standard_normal(out=k[slot], dtype=np.float32)
        g.standard_normal(out=q[slot], dtype=np.float32)
        g.standard_normal(out=v[slot], dtype=np.float32)
        logt = g.uniform(np.log(t_lo), np.log(t_hi), size=N)
        t = np.exp(logt).astype(np.float32)
        q[slot] += pe
        q[slot] *= t[:, None]
        k[slot] += pe

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(one, enumerate(heads)))
    return q, k, v


def entropy_like(seed: int, outer: int, N: int) -> np.ndarray:
    """float32 [outer][N] values spread over [0, ln N] the way attention entropies of the
    generator above spread (most near ln N, a long tail down to 0): a 70/30 mixture of
    ln N - Exp(1.2) and U(0, ln N), clipped to [0, ln N].  Only an input for mask tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED + 1000 + seed)))
    top = np.log(N)
    a = top - g.exponential(1.2, size=(outer, N))
    b = g.uniform(0.0, top, size=(outer, N))
    pick = g.uniform(size=(outer, N)) < 0.7
    return np.clip(np.where(pick, a, b), 0.0, top).astype(np.float32)


def uniform_ints(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Seeded sample of n distinct ints in [lo, hi) (sorted), for sampled parity checks."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED + 2000 + seed)))
    n = min(n, hi - lo)
    return np.sort(g.choice(np.arange(lo, hi), size=n, replace=False)).astype(np.int32)


def normal_chunk(seed: int, which: int, chunk: int, rows: int, D: int) -> np.ndarray:
    """Seeded N(0, 1) float32 [rows][D]: chunk `chunk` of tensor `which` (its own child stream,
    SeedSequence(root + 3000 + seed, spawn_key=(which, chunk))), so any chunk of a very large
    tensor can be drawn alone and chunks can be drawn in parallel."""
    ss = np.random.SeedSequence(ROOT_SEED + 3000 + seed, spawn_key=(which, chunk))
    out = np.empty((rows, D), dtype=np.float32)
    np.random.Generator(np.random.PCG64(ss)).standard_normal(out=out, dtype=np.float32)
    return out


def normal_rows(seed: int, which: int, N: int, D: int, chunk_rows: int = 1 << 18):
    """Tensor `which` of N(0, 1) float32 rows [N][D] in chunks of chunk_rows rows (the last one
    shorter): yields (first_row, chunk) in row order, drawing up to 16 chunks at a time in
    parallel.  Chunk c is normal_chunk(seed, which, c, ...)."""
    starts = list(range(0, N, chunk_rows))
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        for i in range(0, len(starts), _threads()):
            batch = starts[i:i + _threads()]
            arrs = ex.map(lambda s: normal_chunk(seed, which, s // chunk_rows, min(chunk_rows, N - s), D), batch)
            for s, a in zip(batch, arrs):
                yield s, a
