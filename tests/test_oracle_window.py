"""Pins of the oracle's 1D-distance variant of the support ("Token Radius Attention for
Efficient Video Generation", section 4, ablation study: the radius mask replaced by a 1D
distance).

Reading: the budget K_i = tau * exp(H_i) (section 2, Insight I) is spent on a window of the
flattened token sequence in natural raster order n = (f*H + h)*W + w, centred on the query:
key j is kept iff 2 |n_i - n_j| <= K_i.  The oracle evaluates it canonically as d == 0 or
ln d <= (double)H_i + (ln tau - ln 2) through an fp64 table of ln t.  The pins below reach
the same sets by other routes: exp and floor in fp64, counting, brute force over the natural
order, and invariances.
"""
import math

import numpy as np
import pytest


def _natural(orc, F, H, W, th, tw):
    return orc.tile_major_order(F, H, W, th, tw)


def _half_window(H, tau):
    """largest t with 2 t <= tau e^H, by exp and floor (no tables): the window's half-width"""
    if math.isnan(H) or H == -math.inf:
        return 0
    if H == math.inf:
        return 1 << 40
    return int(math.floor(tau * math.exp(H) / 2.0))


def _near_tie(H, tau):
    x = float(np.float32(tau)) * math.exp(float(np.float32(H))) / 2.0
    return abs(x - round(x)) < 1e-9 * max(1.0, x)


@pytest.mark.parametrize("F,H,W,th,tw", [(1, 4, 50, 8, 8), (3, 5, 7, 2, 3), (2, 9, 16, 4, 4)])
def test_window_counts_closed_form(orc, F, H, W, th, tw):
    # query at natural index n keeps min(n, T) keys before it, min(N - 1 - n, T) after it and
    # itself, T = floor(K / 2): clipped at the ends of the sequence
    N = F * H * W
    perm = _natural(orc, F, H, W, th, tw)
    tau = 0.05
    rng = np.random.default_rng(3)
    ent = rng.uniform(0.0, math.log(N) + 3.0, size=N).astype(np.float32)
    for i in rng.choice(N, size=25, replace=False):
        Hi = float(ent[i])
        if _near_tie(Hi, tau):
            continue
        T = _half_window(float(np.float32(Hi)), float(np.float32(tau)))
        n = int(perm[i])
        expect = min(n, T) + min(N - 1 - n, T) + 1
        row = orc.member_row_1d(ent, F, H, W, tau, int(i), th, tw)
        assert int(row.sum()) == expect, (i, Hi, T)
        # and the members are exactly the natural indices within T of n
        nat = np.sort(perm[row.astype(bool)])
        assert np.array_equal(nat, np.arange(max(0, n - T), min(N - 1, n + T) + 1))


def test_window_holds_the_budget(orc):
    # away from the ends of the sequence the window holds 2 floor(K/2) + 1 keys, i.e. K - 1 to
    # K + 1 keys: the budget of Insight I
    F, H, W = 1, 40, 64
    N = F * H * W
    i_mid = int(np.nonzero(_natural(orc, F, H, W, 8, 8) == N // 2)[0][0])
    for tau in (0.01, 0.1, 1.0):
        for Hv in (3.0, 5.5, 7.25):
            ent = np.full(N, Hv, dtype=np.float32)
            K = float(np.float32(tau)) * math.exp(float(np.float32(Hv)))
            cnt = int(orc.member_row_1d(ent, F, H, W, tau, i_mid).sum())
            assert K - 1.0 <= cnt <= K + 1.0, (tau, Hv, K, cnt)


def test_window_special_values(orc):
    # K < 2 keeps the query alone (and so do NaN and -inf); +inf keeps every key
    F, H, W = 2, 6, 8
    N = F * H * W
    ent = np.zeros(N, dtype=np.float32)
    tau = 1.0
    ent[5] = math.log(1.99)      # K = 1.99: T = 0
    ent[6] = math.log(2.01)      # K = 2.01: T = 1
    ent[7] = np.nan
    ent[8] = -np.inf
    ent[9] = np.inf
    perm = _natural(orc, F, H, W, 8, 8)
    assert orc.member_row_1d(ent, F, H, W, tau, 5).sum() == 1
    row = orc.member_row_1d(ent, F, H, W, tau, 6)
    assert row.sum() == 1 + (perm[6] > 0) + (perm[6] < N - 1)
    assert orc.member_row_1d(ent, F, H, W, tau, 7).sum() == 1
    assert orc.member_row_1d(ent, F, H, W, tau, 8).sum() == 1
    assert orc.member_row_1d(ent, F, H, W, tau, 9).sum() == N
    assert orc.window_mu(1.0) == -math.log(2.0)


def test_window_symmetric_and_tile_independent(orc):
    # the support depends on natural indices only: the same natural tokens for every tile shape,
    # and symmetric about the query wherever both sides exist
    F, H, W = 3, 7, 10
    N = F * H * W
    rng = np.random.default_rng(5)
    ent_nat = rng.uniform(0.0, 6.0, size=N).astype(np.float32)   # by natural index
    tau = 0.3
    ref = None
    for th, tw in ((8, 8), (1, 1), (3, 4), (7, 10)):
        perm = _natural(orc, F, H, W, th, tw)
        ent = ent_nat[perm]                                        # tile-major order
        sets = []
        for n in (0, 17, 105, N - 1):
            i = int(np.nonzero(perm == n)[0][0])
            members = np.sort(perm[orc.member_row_1d(ent, F, H, W, tau, i, th, tw).astype(bool)])
            sets.append(members)
            left, right = n - members[0], members[-1] - n
            if members[0] > 0 and members[-1] < N - 1:
                assert left == right
            assert np.array_equal(members, np.arange(members[0], members[-1] + 1))  # contiguous
        if ref is None:
            ref = sets
        for a, b in zip(sets, ref):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("F,H,W,tau,th,tw", [(2, 5, 7, 0.05, 8, 8), (3, 4, 6, 0.5, 2, 3), (1, 9, 13, 1.0, 4, 4)])
def test_window_canonical_equals_direct(orc, F, H, W, tau, th, tw):
    # the table test (ln d <= H + ln tau - ln 2) and the direct test (2 d <= tau e^H) agree on
    # every (query, key) pair
    N = F * H * W
    rng = np.random.default_rng(F + H + W)
    ent = rng.uniform(-1.0, math.log(N) + 2.0, size=N).astype(np.float32)
    assert orc.naive_disagreements_1d(ent, F, H, W, tau, th, tw) == 0


def test_window_nesting(orc):
    # a larger entropy or tau never drops a key
    F, H, W = 2, 8, 12
    N = F * H * W
    rng = np.random.default_rng(9)
    ent = rng.uniform(0.0, 5.0, size=N).astype(np.float32)
    for i in (0, 50, N - 1):
        a = orc.member_row_1d(ent, F, H, W, 0.1, i)
        b = orc.member_row_1d(ent, F, H, W, 0.3, i)
        assert np.all(b >= a)
        e2 = ent.copy()
        e2[i] += 0.7
        c = orc.member_row_1d(e2, F, H, W, 0.1, i)
        assert np.all(c >= a)


@pytest.mark.parametrize("bq,bk,vote", [(64, 64, 1), (32, 16, 1), (32, 16, 3)])
def test_window_block_voting(orc, bq, bk, vote):
    # votes(Qb, Kb) = number of queries of Qb whose window meets Kb (from the member rows);
    # retained iff votes >= threshold or Kb overlaps Qb's range; threshold 1 = OR of the token mask
    F, H, W, tau = 2, 9, 14, 0.2
    N = F * H * W
    rng = np.random.default_rng(bq + bk + vote)
    ent = rng.uniform(0.0, math.log(N), size=N).astype(np.float32)
    mask, votes = orc.block_mask_1d(ent, F, H, W, tau, bq, bk, vote)
    nqb, nkb = -(-N // bq), -(-N // bk)
    rows = np.stack([orc.member_row_1d(ent, F, H, W, tau, i) for i in range(N)])
    for qb in range(nqb):
        q0, q1 = qb * bq, min(N, qb * bq + bq)
        for kb in range(nkb):
            k0, k1 = kb * bk, min(N, kb * bk + bk)
            v = int(np.sum(rows[q0:q1, k0:k1].any(axis=1)))
            assert votes[qb, kb] == v
            diag = k0 < q1 and q0 < k1
            assert mask[qb, kb] == (v >= vote or diag)
    if vote == 1:
        tok = np.stack([rows[qb * bq:(qb + 1) * bq].any(axis=0) for qb in range(nqb)])
        blk = np.stack([[tok[qb, kb * bk:(kb + 1) * bk].any() for kb in range(nkb)] for qb in range(nqb)])
        assert np.array_equal(mask.astype(bool), blk)


def test_window_block_mask_selected_rows(orc):
    # the rows of selected q-blocks equal the same rows of the full mask
    F, H, W, tau = 3, 10, 16, 0.05
    N = F * H * W
    ent = np.random.default_rng(2).uniform(0.0, math.log(N), size=N).astype(np.float32)
    full, _ = orc.block_mask_1d(ent, F, H, W, tau, 64, 64)
    sel = np.array([0, 3, 7], dtype=np.int32)
    part, _ = orc.block_mask_1d(ent, F, H, W, tau, 64, 64, qblocks=sel)
    assert np.array_equal(part, full[sel])
