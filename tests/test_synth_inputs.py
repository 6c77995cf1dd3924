"""The seeded inputs have the property the method rests on ("Token Radius Attention for
Efficient Video Generation", section 2, Insight I): a query's attention entropy predicts
how many keys carry its mass, so a budget proportional to exp(H) follows the keys a query
actually needs.  Checked on the tiny workload's seeded q, k (fp64 softmax in numpy): the
entropies span most of [0, ln N], and log of the number of keys holding 90% of each row's
mass rises with H (rank correlation close to 1)."""
import math

import numpy as np

from entropy_adaptive_sparse_amd import synth, workloads


def _rank(x):
    r = np.empty(len(x))
    r[np.argsort(x)] = np.arange(len(x))
    return r


def test_entropy_predicts_effective_key_count():
    wl = workloads.get(1)
    q, k, _ = synth.qkv(wl.wid, wl.outer, wl.F, wl.H, wl.W, wl.D, wl.t_lo, wl.t_hi, heads=[0])
    s = (q[0].astype(np.float64) @ k[0].astype(np.float64).T) * wl.sm_scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    H = -(p * np.log(np.where(p > 0, p, 1.0))).sum(axis=1)
    srt = -np.sort(-p, axis=1)
    k90 = (np.cumsum(srt, axis=1) < 0.9).sum(axis=1) + 1
    assert H.min() < 0.2 * math.log(wl.N) and H.max() > 0.9 * math.log(wl.N)
    rho = np.corrcoef(_rank(H), _rank(np.log(k90)))[0, 1]
    assert rho > 0.95, rho
    # and the budget exp(H) is within a constant factor of k90 for most queries
    ratio = np.log(k90) - H
    assert np.percentile(ratio, 95) - np.percentile(ratio, 5) < 2.5


def test_normal_rows_chunks_are_reproducible_and_independent():
    # the chunked generator behind the largest-head tests: every chunk is normal_chunk drawn
    # alone (so a test can redraw any rows it checks), chunks and tensors differ, and the values
    # are standard normal
    N, D, rows = 1000, 8, 96
    got = list(synth.normal_rows(5, 1, N, D, chunk_rows=rows))
    assert [s for s, _ in got] == list(range(0, N, rows))
    assert sum(a.shape[0] for _, a in got) == N and all(a.dtype == np.float32 for _, a in got)
    for s, a in got:
        assert np.array_equal(a, synth.normal_chunk(5, 1, s // rows, min(rows, N - s), D))
    full = np.concatenate([a for _, a in got])
    again = np.concatenate([a for _, a in synth.normal_rows(5, 1, N, D, chunk_rows=rows)])
    assert np.array_equal(full, again)
    other = np.concatenate([a for _, a in synth.normal_rows(5, 2, N, D, chunk_rows=rows)])
    assert not np.array_equal(full, other)
    assert not np.array_equal(got[0][1], got[1][1][:rows])
    assert abs(float(full.mean())) < 0.05 and abs(float(full.std()) - 1.0) < 0.05
