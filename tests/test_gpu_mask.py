"""GPU parity: entropy -> budget -> radius -> block-sparse mask, bit-exact against the
oracle's brute-force (query, key) disk test and token voting ("Token Radius Attention
for Efficient Video Generation", section 2: Insight I, Insight II, TRA pipeline steps
2-3).  Both sides take the same fp32 entropy array (from the seeded generator, or the
oracle's own fp64 entropies rounded to fp32) and the same fp32 tau and gamma."""

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import device, qkv_inputs, say, sample_rows, small_workload, torch_mod, tra

pytestmark = pytest.mark.gpu


def _gpu_mask(t, ent, F, H, W, tau, gamma, bq, bk, vote, th=8, tw=8):
    torch = torch_mod()
    e = torch.from_numpy(np.ascontiguousarray(ent)).to(device())
    cnt, idx, msk = t.build_block_mask(e, F, H, W, tau, gamma, bq, bk, vote, th, tw, want_mask=True)
    torch.cuda.synchronize()
    return cnt.cpu().numpy(), idx.cpu().numpy(), msk.cpu().numpy()


def _compare(orc, ent, cnt, idx, msk, F, H, W, tau, gamma, bq, bk, vote, heads, qblocks=None, th=8, tw=8):
    for h in heads:
        ref, _ = orc.block_mask(ent[h], F, H, W, tau, gamma, bq, bk, vote, th, tw, qblocks=qblocks)
        sel = np.arange(ref.shape[0]) if qblocks is None else np.asarray(qblocks)
        assert np.array_equal(msk[h][sel], ref), "head %d mask" % h
        rc, lists = orc.mask_to_lists(ref)
        assert np.array_equal(cnt[h][sel], rc), "head %d kv_count" % h
        for s, qb in enumerate(sel):
            assert np.array_equal(idx[h, qb, :rc[s]], lists[s]), "head %d qb %d kv_index" % (h, qb)


@pytest.mark.parametrize("F,H,W,tau,gamma,bq,vote", [
    (4, 16, 16, 1.0, 0.5, 64, 1),      # tiny workload, tau = 1
    (4, 16, 16, 0.01, 0.5, 64, 1),
    (4, 16, 16, 0.03, 0.5, 128, 1),
    (4, 16, 16, 0.03, 0.5, 128, 2),
    (4, 16, 16, 0.03, 0.5, 64, 8),
    (3, 15, 17, 0.02, 0.0, 128, 1),    # ragged blocks and tiles, no temporal decay
    (5, 9, 22, 0.2, 1.5, 64, 3),
    (2, 45, 80, 0.03, 0.5, 128, 1),    # two frames of the 720p grid
    (12, 5, 7, 0.05, 0.3, 128, 1),     # frames smaller than a q-block: up to five frames per q-block
    (12, 5, 7, 0.05, 0.3, 64, 2),
    (7, 11, 3, 0.5, 0.2, 128, 1),      # columns narrower than a tile
    (40, 2, 3, 0.3, 0.1, 128, 1),      # 6-token frames: a k-block spans a dozen frames
    (9, 13, 11, 0.05, 0.4, 64, 2),
])
def test_mask_small_all_blocks(orc, F, H, W, tau, gamma, bq, vote):
    t = tra()
    N = F * H * W
    say("mask small", F, H, W, tau, gamma, bq, vote)
    ent = synth.entropy_like(F * 7 + H, 2, N)
    cnt, idx, msk = _gpu_mask(t, ent, F, H, W, tau, gamma, bq, 64, vote)
    _compare(orc, ent, cnt, idx, msk, F, H, W, tau, gamma, bq, 64, vote, heads=range(2))


@pytest.mark.parametrize("bq", [128, 64])
def test_mask_largest_frame_count(orc, bq):
    # the most frames the builder's LDS holds for this block_q (per-query thresholds toward every
    # frame): found by asking the library, which refuses one frame more before any launch; that
    # grid bit for bit against the oracle, every q-block of both heads
    t = tra()
    H, W, tau, gamma = 2, 3, 0.3, 0.2
    F = 1
    while True:
        try:
            t.mask_prepare(F + 1, H, W, tau, gamma, bq, 64)
        except t.TraError as e:
            assert e.code == 2, "expected TRA_ERR_UNSUPPORTED past the largest frame count"
            break
        F += 1
        assert F < 4096
    say("mask at the largest frame count", F, "frames, block_q", bq)
    assert F >= 40
    ent = synth.entropy_like(960 + bq, 2, F * H * W)
    cnt, idx, msk = _gpu_mask(t, ent, F, H, W, tau, gamma, bq, 64, 1)
    _compare(orc, ent, cnt, idx, msk, F, H, W, tau, gamma, bq, 64, 1, heads=range(2))


@pytest.mark.parametrize("tile", [(1, 1), (3, 5), (4, 16), (16, 16), (2, 8)])
@pytest.mark.parametrize("F,H,W,tau,gamma,bq,vote", [
    (4, 16, 16, 0.03, 0.5, 128, 1),
    (3, 15, 17, 0.02, 0.3, 64, 2),     # clipped tiles on both edges
    (6, 9, 22, 0.1, 0.5, 128, 1),
])
def test_mask_tile_shapes(orc, tile, F, H, W, tau, gamma, bq, vote):
    # the k-block rectangles, the reach windows (rounded out to whole tiles) and the tile-major
    # ranges all depend on the tile shape: every q-block of both heads, bit for bit
    t = tra()
    N = F * H * W
    th, tw = tile
    say("mask tile shape", tile, F, H, W, tau, gamma, bq, vote)
    ent = synth.entropy_like(F * 11 + W + th, 2, N)
    cnt, idx, msk = _gpu_mask(t, ent, F, H, W, tau, gamma, bq, 64, vote, th, tw)
    _compare(orc, ent, cnt, idx, msk, F, H, W, tau, gamma, bq, 64, vote, heads=range(2), th=th, tw=tw)


@pytest.mark.parametrize("bq,vote", [(128, 1), (64, 1), (128, 3)])
def test_mask_special_entropies(orc, bq, vote):
    # NaN and -inf reach only distance 0, +inf the whole frame; negative, zero and
    # large finite entropies mixed in, whole frames of NaN included
    F, H, W = 4, 24, 40
    N = F * H * W
    say("mask special entropies", bq, vote)
    ent = synth.entropy_like(55, 2, N)
    rng = np.random.default_rng(56)
    pick = rng.random(ent.shape)
    ent[pick < 0.05] = np.nan
    ent[(pick >= 0.05) & (pick < 0.07)] = -np.inf
    ent[(pick >= 0.075) & (pick < 0.15)] *= -1.0
    ent[(pick >= 0.15) & (pick < 0.2)] = 0.0
    ent[(pick >= 0.2) & (pick < 0.205)] = 9.5
    ent[1, 2 * H * W:3 * H * W] = np.nan
    ent[0, 17] = np.inf
    ent[1, 700] = np.inf
    t = tra()
    for tau in (0.02, 0.002):
        cnt, idx, msk = _gpu_mask(t, ent, F, H, W, tau, 0.5, bq, 64, vote)
        _compare(orc, ent, cnt, idx, msk, F, H, W, tau, 0.5, bq, 64, vote, heads=range(2))


def test_mask_from_oracle_entropies_tiny(orc):
    # the real pipeline on the tiny workload: the oracle's fp64 entropies of the seeded
    # q, k, v (rounded to fp32, in tile-major order) feed both mask builders
    wl = workloads.get(1)
    t = tra()
    q, k, v = qkv_inputs(wl)
    perm = orc.tile_major_order(wl.F, wl.H, wl.W)
    ent = np.empty((wl.outer, wl.N), dtype=np.float32)
    for h in range(wl.outer):
        _, H, _ = orc.attention(q[h].numpy(), k[h].numpy(), v[h].numpy())
        ent[h] = H[perm].astype(np.float32)
    for tau in (1.0, 0.03, 0.01):
        say("mask tiny oracle entropies tau", tau)
        cnt, idx, msk = _gpu_mask(t, ent, wl.F, wl.H, wl.W, tau, wl.gamma, wl.block_q, wl.block_k, 1)
        _compare(orc, ent, cnt, idx, msk, wl.F, wl.H, wl.W, tau, wl.gamma, wl.block_q, wl.block_k, 1,
                 heads=range(wl.outer))


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_mask_full_size_sampled(orc, wid):
    # full geometry and every head on the GPU; the oracle checks seeded q-blocks of
    # seeded heads (every head's ragged last q-block included)
    wl = workloads.get(wid)
    t = tra()
    say("mask full size workload", wid, wl.name, "tau", wl.tau)
    ent = synth.entropy_like(100 + wid, wl.outer, wl.N)
    cnt, idx, msk = _gpu_mask(t, ent, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k,
                              wl.vote_threshold)
    blocks, _ = sample_rows(wid, wl.N, wl.block_q, 4)
    heads = synth.uniform_ints(wid, 3, 0, wl.outer)
    _compare(orc, ent, cnt, idx, msk, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k,
             wl.vote_threshold, heads=heads, qblocks=blocks)
    # structural checks on every row: ascending, in range, counts consistent with the byte mask
    assert np.array_equal(cnt, msk.sum(axis=2))
    nkb = wl.nkb
    for h in range(wl.outer):
        for qb in range(0, wl.nqb, 37):
            row = idx[h, qb, :cnt[h, qb]]
            assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < nkb
    dens = msk.mean()
    say("  block density (unweighted)", float(dens))


def test_mask_deterministic_and_reusable(orc):
    # the mask is a pure function of (entropy, geometry, tau, gamma, blocks, vote, tile)
    t = tra()
    F, H, W = 6, 30, 52
    ent = synth.entropy_like(7, 3, F * H * W)
    a = _gpu_mask(t, ent, F, H, W, 0.01, 0.5, 128, 64, 1)
    b = _gpu_mask(t, ent, F, H, W, 0.01, 0.5, 128, 64, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_mask_capacity_error():
    # the binding refuses a kv_index of the wrong shape; the C ABI refuses a capacity below
    # outer * nqb * nkb with TRA_ERR_CAPACITY, before any HIP call
    torch = torch_mod()
    t = tra()
    e = torch.zeros((1, 1024), device=device())
    cnt = torch.empty((1, 16), dtype=torch.int32, device=device())
    idx = torch.empty((1, 16, 15), dtype=torch.int32, device=device())
    with pytest.raises(ValueError):
        t.build_block_mask(e, 4, 16, 16, 1.0, 0.5, 64, 64, 1, kv_count=cnt, kv_index=idx)
    rc = t.load().tra_build_block_mask(e.data_ptr(), 1, 4, 16, 16, 1.0, 0.5, 64, 64, 1, 8, 8, cnt.data_ptr(),
                                       idx.data_ptr(), idx.numel(), None, None)
    assert rc == 4


def test_mask_end_to_end_own_entropies(orc):
    # each side from its own entropies: the GPU's dense pass feeds the GPU mask builder, the
    # oracle's fp64 entropies (rounded to fp32) feed the oracle's.  Entropies differ within
    # the 1e-3 nats tolerance, so a query whose disk edge sits on a lattice point can flip a
    # block: the agreement is a statistic; the bound here only catches a systematic error.
    torch = torch_mod()
    t = tra()
    wl = small_workload(77, 4, 24, 40, 128, "bf16", outer=2, tau=0.03)
    q, k, v = qkv_inputs(wl)
    qp, kp, vp = (t.tile_major_permute(x.to(device()), wl.F, wl.H, wl.W) for x in (q, k, v))
    _, eg, _ = t.dense_attn_entropy(qp, kp, vp, wl.sm_scale, entropy=True)
    torch.cuda.synchronize()
    ent_gpu = eg.cpu().numpy()
    cnt, idx, msk = _gpu_mask(t, ent_gpu, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k, 1)
    perm = orc.tile_major_order(wl.F, wl.H, wl.W)
    differ = total = 0
    worst_ent = 0.0
    for h in range(wl.outer):
        _, Hh, _ = orc.attention(q[h].float().numpy(), k[h].float().numpy(), v[h].float().numpy(), wl.sm_scale)
        ent_orc = Hh[perm].astype(np.float32)
        worst_ent = max(worst_ent, float(np.max(np.abs(ent_orc - ent_gpu[h]))))
        ref, _ = orc.block_mask(ent_orc, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k, 1)
        differ += int(np.sum(ref != msk[h]))
        total += ref.size
    say("  entropy max diff %.2e nats; mask entries differing %d of %d (%.3f%%)"
        % (worst_ent, differ, total, 100.0 * differ / total))
    assert worst_ent <= 1e-3
    assert differ <= 0.01 * total
