"""Pins of the oracle's budget, radius, disk, tile-major order and block voting.

Readings follow "Token Radius Attention for Efficient Video Generation" (gist.science
summary of arXiv 2608.02504), section 2: Insight I (budget tau * exp(H_i) / N),
Insight II (budget -> radius, temporal factor phi(delta) = exp(-gamma delta)) and the
TRA pipeline (2D disk per frame; tile-major layout; fused distance / radius compare /
block pruning / token voting into a block-sparse mask).
"""
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t) for t in line.split()])
    return rows


# ------------------------------------------------------------------ budget and radius
def test_budget_closed_forms(orc):
    # a uniform row over N keys has H = ln N: with tau = 1 the budget is all N keys;
    # a one-hot row has H = 0: the budget is tau tokens
    for N in (1024, 32760, 75600):
        assert abs(orc.token_budget(math.log(N), 1.0) - N) < 1e-9 * N
    for tau in (0.01, 0.5, 3.0):
        assert orc.token_budget(0.0, tau) == tau


@pytest.mark.parametrize("F,gamma", [(1, 0.5), (4, 0.5), (21, 0.5), (33, 0.25), (7, 0.0), (5, 2.0)])
def test_frame_norm_geometric_closed_form(orc, F, gamma):
    S = orc.frame_norm(F, gamma)
    a = math.exp(-2.0 * gamma)
    for f in range(F):
        if gamma == 0.0:
            ref = float(F)
        else:
            ref = (1 - a ** (f + 1)) / (1 - a) + (1 - a ** (F - f)) / (1 - a) - 1.0
        assert abs(S[f] - ref) < 1e-12 * max(1.0, ref)


def test_area_matching_radius(orc):
    # the per-frame disks rho(f') = r exp(-gamma |f - f'|) have total area K
    F, gamma, tau = 21, 0.5, 0.03
    S = orc.frame_norm(F, gamma)
    for H in (0.5, 4.0, 11.0):
        for f in (0, 7, 20):
            r = orc.base_radius(H, tau, S[f])
            area = sum(math.pi * (r * math.exp(-gamma * abs(f - g))) ** 2 for g in range(F))
            assert abs(area - tau * math.exp(H)) < 1e-9 * tau * math.exp(H)


def test_lambda_table_properties(orc):
    F = 9
    lam0 = orc.lambda_table(F, 0.03, 0.0)
    assert np.all(lam0 == lam0[:, :1])  # gamma = 0: no dependence on the key frame
    lam = orc.lambda_table(F, 0.03, 0.5)
    for f in range(F):
        d = np.abs(np.arange(F) - f)
        order = np.argsort(d, kind="stable")
        vals = lam[f][order]
        assert np.all(np.diff(vals)[np.diff(d[order]) > 0] < 0)  # strictly shrinking with delta
    # ln tau enters additively
    lam2 = orc.lambda_table(F, 0.3, 0.5)
    assert np.allclose(lam2 - lam, math.log(np.float32(0.3)) - math.log(np.float32(0.03)), atol=1e-12)


def test_log_table(orc):
    t = orc.log_table(100)
    assert t[0] == -np.inf and t[1] == 0.0
    assert abs(t[100] - 2 * math.log(10)) < 1e-15
    assert np.all(np.diff(t[1:]) > 0)


# ------------------------------------------------------------------ disk
def _center_row(orc, T, side=41):
    # one frame, identity tiles, gamma = 0, tau = pi (as fp32): threshold s = H + ln(tau/pi)
    # sits inside [ln T, ln(T+1)) when H = ln(T + 1/2)
    H = np.float32(math.log(T + 0.5)) if T > 0 else np.float32(math.log(0.5))
    ent = np.full(side * side, H, dtype=np.float32)
    c = (side // 2) * side + side // 2
    return orc.member_row(ent, 1, side, side, float(np.float32(math.pi)), 0.0, c, th=1, tw=1).reshape(side, side)


def test_disk_lattice_counts(orc):
    for T, count in _golden_rows("gauss_circle_counts.txt"):
        row = _center_row(orc, T)
        assert int(row.sum()) == count, (T, int(row.sum()), count)


def test_disk_symmetry(orc):
    for T in (5, 13, 40, 100):
        m = _center_row(orc, T)
        assert np.array_equal(m, m[::-1, :]) and np.array_equal(m, m[:, ::-1]) and np.array_equal(m, m.T)


def _tiny_geometry_cases():
    return [(3, 7, 9, 0.05, 0.5, 4, 4), (2, 8, 8, 0.3, 0.0, 8, 8), (4, 5, 6, 1.0, 0.5, 2, 3),
            (5, 6, 5, 0.01, 1.3, 3, 2)]


def test_canonical_table_test_matches_direct_radius_test(orc):
    r = np.random.default_rng(11)
    for F, H, W, tau, gamma, th, tw in _tiny_geometry_cases():
        N = F * H * W
        ent = r.uniform(0, math.log(N), size=N).astype(np.float32)
        assert orc.naive_disagreements(ent, F, H, W, tau, gamma, th, tw) == 0


def test_radius_shrinks_with_temporal_distance_and_temporal_column(orc):
    F, H, W = 7, 16, 16
    perm = orc.tile_major_order(F, H, W)
    pos_of = np.empty_like(perm)
    pos_of[perm] = np.arange(F * H * W)
    for tau, H_i in ((0.05, 6.0), (1.0, 4.0)):
        ent = np.full(F * H * W, np.float32(H_i), dtype=np.float32)
        nat_i = (3 * H + 8) * W + 8
        i = int(pos_of[nat_i])
        row = orc.member_row(ent, F, H, W, tau, 0.5, i)
        per_frame = np.zeros(F, dtype=int)
        nat = perm[np.nonzero(row)[0]]
        for n in nat:
            per_frame[n // (H * W)] += 1
        for d in range(1, 4):
            assert per_frame[3 + d] <= per_frame[3 + d - 1] and per_frame[3 - d] <= per_frame[3 - d + 1]
        assert per_frame[3] > per_frame[0]
        for f in range(F):  # the co-located key of every frame is always kept
            assert row[pos_of[(f * H + 8) * W + 8]] == 1


def test_support_nested_in_entropy_and_tau(orc):
    F, H, W = 3, 12, 12
    N = F * H * W
    i = 200
    prev = None
    for Hv in (0.0, 1.0, 2.5, 4.0, 6.0):
        row = orc.member_row(np.full(N, Hv, np.float32), F, H, W, 0.05, 0.5, i)
        if prev is not None:
            assert np.all(row >= prev)
        prev = row
    prev = None
    for tau in (0.001, 0.01, 0.1, 1.0):
        row = orc.member_row(np.full(N, 3.0, np.float32), F, H, W, tau, 0.5, i)
        if prev is not None:
            assert np.all(row >= prev)
        prev = row


# ------------------------------------------------------------------ tile-major order
def test_tile_major_golden(orc):
    (expected,) = _golden_rows("perm_F1_H3_W5_t2x2.txt")
    assert orc.tile_major_order(1, 3, 5, 2, 2).tolist() == expected


@pytest.mark.parametrize("F,H,W", [(1, 1, 1), (4, 16, 16), (2, 30, 52), (2, 45, 80), (3, 9, 9)])
def test_tile_major_identity_cases_and_bijection(orc, F, H, W):
    ident = np.arange(F * H * W)
    for th, tw in ((1, 1), (1, W), (H, W)):
        assert np.array_equal(orc.tile_major_order(F, H, W, th, tw), ident)
    perm = orc.tile_major_order(F, H, W, 8, 8)
    assert np.array_equal(np.sort(perm), ident)
    x = np.random.default_rng(0).standard_normal((F * H * W, 3))
    assert np.array_equal(orc.unpermute(orc.permute(x, perm), perm), x)


def _closed_form(p, F, H, W, th, tw):
    # closed form of the tile-major position -> natural index map (used by the GPU kernels)
    HW = H * W
    f, r = divmod(p, HW)
    ty, r2 = divmod(r, th * W)
    ht = np.minimum(th, H - ty * th)
    tx, r3 = divmod(r2, ht * tw)
    wt = np.minimum(tw, W - tx * tw)
    y = ty * th + r3 // wt
    x = tx * tw + r3 % wt
    return (f * H + y) * W + x


@pytest.mark.parametrize("F,H,W,th,tw", [(4, 16, 16, 8, 8), (2, 30, 52, 8, 8), (2, 45, 80, 8, 8),
                                          (1, 3, 5, 2, 2), (2, 9, 7, 4, 3), (1, 13, 11, 5, 4)])
def test_tile_major_closed_form_equals_enumeration(orc, F, H, W, th, tw):
    perm = orc.tile_major_order(F, H, W, th, tw)
    p = np.arange(F * H * W)
    assert np.array_equal(_closed_form(p, F, H, W, th, tw), perm)


# ------------------------------------------------------------------ blocks and votes
def _geom_case():
    return dict(F=3, H=12, W=20, tau=0.02, gamma=0.5, bq=64, bk=32)  # N = 720: ragged blocks


def test_threshold_one_is_or_of_token_mask_and_votes_count_queries(orc):
    g = _geom_case()
    F, H, W, bq, bk = g["F"], g["H"], g["W"], g["bq"], g["bk"]
    N = F * H * W
    ent = np.random.default_rng(12).uniform(0, math.log(N), N).astype(np.float32)
    nqb, nkb = -(-N // bq), -(-N // bk)
    mask, votes = orc.block_mask(ent, F, H, W, g["tau"], g["gamma"], bq, bk, 1)
    for qb in range(nqb):
        ref_votes = np.zeros(nkb, dtype=int)
        for i in range(qb * bq, min(N, qb * bq + bq)):
            row = orc.member_row(ent, F, H, W, g["tau"], g["gamma"], i)
            touched = np.zeros(nkb, dtype=bool)
            touched[np.nonzero(row)[0] // bk] = True
            ref_votes += touched
        assert np.array_equal(votes[qb], ref_votes)
        assert np.array_equal(mask[qb], (ref_votes >= 1).astype(np.uint8))


def test_threshold_monotone_and_diagonal_kept(orc):
    g = _geom_case()
    F, H, W, bq, bk = g["F"], g["H"], g["W"], g["bq"], g["bk"]
    N = F * H * W
    ent = np.random.default_rng(13).uniform(0, math.log(N), N).astype(np.float32)
    prev = None
    for vt in (1, 2, 8, 32, 10 ** 6):
        m, votes = orc.block_mask(ent, F, H, W, g["tau"], g["gamma"], bq, bk, vt)
        if prev is not None:
            assert np.all(m <= prev)
        prev = m
        for qb in range(m.shape[0]):
            for kb in range(m.shape[1]):
                if kb * bk < min(N, qb * bq + bq) and qb * bq < min(N, kb * bk + bk):
                    assert m[qb, kb] == 1
    # an impossible threshold leaves only the diagonal
    nd = sum(1 for qb in range(prev.shape[0]) for kb in range(prev.shape[1])
             if kb * bk < min(N, qb * bq + bq) and qb * bq < min(N, kb * bk + bk))
    assert int(prev.sum()) == nd


def test_saturation_keeps_every_block(orc):
    F, H, W = 2, 16, 16
    N = F * H * W
    ent = np.full(N, np.float32(math.log(N)), dtype=np.float32)
    m, _ = orc.block_mask(ent, F, H, W, 1.0e6, 0.0, 64, 64, 1)
    assert np.all(m == 1)


def test_sampled_rows_match_full(orc):
    g = _geom_case()
    F, H, W, bq, bk = g["F"], g["H"], g["W"], g["bq"], g["bk"]
    N = F * H * W
    ent = np.random.default_rng(14).uniform(0, math.log(N), N).astype(np.float32)
    full, fv = orc.block_mask(ent, F, H, W, g["tau"], g["gamma"], bq, bk, 2)
    sel = np.array([10, 0, 5], dtype=np.int32)
    part, pv = orc.block_mask(ent, F, H, W, g["tau"], g["gamma"], bq, bk, 2, qblocks=sel)
    assert np.array_equal(part, full[sel]) and np.array_equal(pv, fv[sel])
    counts, lists = orc.mask_to_lists(part)
    for c, lst in zip(counts, lists):
        assert len(lst) == c and np.all(np.diff(lst) > 0)
