"""GPU parity: the 1D-distance variant of the mask ("Token Radius Attention for Efficient Video
Generation", section 4, ablation study: the radius mask replaced by a 1D distance), bit-exact
against the oracle's brute force over every (query, key) pair: the budget tau * exp(H_i) spent on
a window of the natural raster sequence, 2 |n_i - n_j| <= K_i, voted into blocks.  Both sides take
the same fp32 entropies (seeded generator) and the same fp32 tau."""
import math

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import device, sample_rows, say, torch_mod, tra

pytestmark = pytest.mark.gpu


def _gpu(t, ent, F, H, W, tau, bq, vote, th=8, tw=8):
    torch = torch_mod()
    e = torch.from_numpy(np.ascontiguousarray(ent)).to(device())
    cnt, idx, msk = t.build_block_mask_1d(e, F, H, W, tau, bq, 64, vote, th, tw, want_mask=True)
    torch.cuda.synchronize()
    return cnt.cpu().numpy(), idx.cpu().numpy(), msk.cpu().numpy()


def _compare(orc, ent, cnt, idx, msk, F, H, W, tau, bq, vote, heads, qblocks=None, th=8, tw=8):
    for h in heads:
        ref, _ = orc.block_mask_1d(ent[h], F, H, W, tau, bq, 64, vote, th, tw, qblocks=qblocks)
        sel = np.arange(ref.shape[0]) if qblocks is None else np.asarray(qblocks)
        assert np.array_equal(msk[h][sel], ref), "head %d mask" % h
        rc, lists = orc.mask_to_lists(ref)
        assert np.array_equal(cnt[h][sel], rc), "head %d kv_count" % h
        for s, qb in enumerate(sel):
            assert np.array_equal(idx[h, qb, :rc[s]], lists[s]), "head %d qb %d kv_index" % (h, qb)


@pytest.mark.parametrize("F,H,W,tau,bq,vote,tile", [
    (4, 16, 16, 1.0, 64, 1, (8, 8)),
    (4, 16, 16, 0.03, 128, 1, (8, 8)),
    (4, 16, 16, 0.03, 128, 3, (8, 8)),
    (3, 15, 17, 0.02, 64, 2, (8, 8)),      # ragged blocks and clipped tiles
    (2, 45, 80, 0.03, 128, 1, (8, 8)),
    (12, 5, 7, 0.05, 128, 1, (8, 8)),      # windows spanning frames
    (5, 9, 22, 0.2, 64, 1, (3, 5)),
    (3, 21, 24, 0.01, 128, 1, (1, 1)),     # 1 x 1 tiles: tile-major = natural order
    (2, 30, 52, 0.004, 128, 8, (16, 16)),
    (1, 1, 1, 0.5, 64, 1, (8, 8)),         # one token
])
def test_mask1d_small_all_blocks(orc, F, H, W, tau, bq, vote, tile):
    t = tra()
    N = F * H * W
    say("1d mask", F, H, W, tau, bq, vote, tile)
    ent = synth.entropy_like(F * 5 + W, 2, N)
    cnt, idx, msk = _gpu(t, ent, F, H, W, tau, bq, vote, *tile)
    _compare(orc, ent, cnt, idx, msk, F, H, W, tau, bq, vote, range(2), th=tile[0], tw=tile[1])
    say("  density %.3f" % float(msk.mean()))


def test_mask1d_special_entropies(orc):
    # NaN and -inf keep only the query itself, +inf the whole sequence; negative and zero entropies
    F, H, W = 4, 24, 40
    N = F * H * W
    ent = synth.entropy_like(91, 2, N)
    rng = np.random.default_rng(92)
    pick = rng.random(ent.shape)
    ent[pick < 0.05] = np.nan
    ent[(pick >= 0.05) & (pick < 0.07)] = -np.inf
    ent[(pick >= 0.075) & (pick < 0.15)] *= -1.0
    ent[(pick >= 0.15) & (pick < 0.2)] = 0.0
    ent[0, 17] = np.inf
    t = tra()
    for tau, bq, vote in ((0.02, 128, 1), (0.002, 64, 1), (0.05, 128, 3)):
        say("1d mask special entropies", tau, bq, vote)
        cnt, idx, msk = _gpu(t, ent, F, H, W, tau, bq, vote)
        _compare(orc, ent, cnt, idx, msk, F, H, W, tau, bq, vote, range(2))


@pytest.mark.parametrize("wid", [3, 4])
def test_mask1d_full_size_sampled(orc, wid):
    # every head and q-block on the GPU at the workload's shape and tau; seeded q-blocks (the ragged
    # last one included) of two seeded heads against the oracle; structure checked on every row
    t = tra()
    wl = workloads.get(wid)
    say("1d mask full size", wl.name)
    ent = synth.entropy_like(900 + wid, wl.outer, wl.N)
    t.mask_prepare_1d(wl.F, wl.H, wl.W, wl.tau, wl.block_q, wl.block_k)
    cnt, idx, msk = _gpu(t, ent, wl.F, wl.H, wl.W, wl.tau, wl.block_q, wl.vote_threshold)
    assert np.array_equal(cnt, msk.sum(axis=2))
    blocks, _ = sample_rows(910 + wid, wl.N, wl.block_q, 4)
    heads = synth.uniform_ints(920 + wid, 2, 0, wl.outer)
    _compare(orc, ent, cnt, idx, msk, wl.F, wl.H, wl.W, wl.tau, wl.block_q, wl.vote_threshold, heads, qblocks=blocks)
    say("  density %.4f" % float(msk.mean()))


def test_mask1d_budget_window_on_a_line():
    # a closed form at full size: one frame row W = N (H = F = 1), tile 1 x 1, so natural = tile-major and
    # a q-block of queries all with entropy H keeps the k-blocks within floor(tau e^H / 2) of its range
    torch = torch_mod()
    t = tra()
    F, H, W, tau = 1, 1, 64 * 200, 1.0
    N = F * H * W
    for Hv in (2.0, 5.5, 8.0):
        ent = np.full((1, N), Hv, dtype=np.float32)
        cnt, idx, msk = _gpu(t, ent, F, H, W, tau, 128, 1, 1, 1)
        T = int(math.floor(float(np.float32(tau)) * math.exp(float(np.float32(Hv))) / 2.0))
        for qb in (0, 37, 99):
            lo, hi = max(0, qb * 128 - T), min(N - 1, qb * 128 + 127 + T)
            want = np.zeros(N // 64, dtype=np.uint8)
            want[lo // 64: hi // 64 + 1] = 1
            assert np.array_equal(msk[0, qb], want), (Hv, qb)
