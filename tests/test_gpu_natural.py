"""GPU: the natural-order attention calls (the tile-major permutation of "Token Radius
Attention for Efficient Video Generation", section 2, TRA pipeline step 3, applied inside
the kernels' loads and stores).

Each call is compared
- with the oracle directly: outputs in natural order within the attention tolerances of the
  oracle's fp64 attention (dense, or restricted to the oracle's block mask), entropy and lse
  by tile-major position; the fused warm-up's mask rows between the oracle's bounds
  (gpu_util.mask_bounds) -- on small grids in full and on seeded q-blocks at full size;
- bit for bit with tile-major calls: the sparse call with the permute -> tile-major call ->
  unpermute chain; the dense calls (which sum over the keys in natural order) with the
  tile-major call on permuted q and natural-order k, v, o unpermuted.
"""
import dataclasses

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import (LSE_TOL, check_output, check_warmup_against_oracle, device, np64, qkv_inputs, rows_of_blocks,
                      sample_rows, say, small_workload, torch_mod, tra)

pytestmark = pytest.mark.gpu


def _wl(seed, F, H, W, tile=(8, 8), tau=0.03, outer=2):
    wl = small_workload(seed, F, H, W, 128, "bf16", outer=outer, tau=tau)
    return dataclasses.replace(wl, tile_h=tile[0], tile_w=tile[1])


def _bits(x):
    torch = torch_mod()
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def _compare(t, wl, q, k, v):
    """natural calls vs tile-major calls, bit for bit; returns the natural dense outputs"""
    torch = torch_mod()
    F, H, W, th, tw = wl.F, wl.H, wl.W, wl.tile_h, wl.tile_w
    qp, kp, vp = (t.tile_major_permute(x, F, H, W, th, tw) for x in (q, k, v))
    # dense: the tile-major kernel on permuted q with k, v as given (keys in natural order)
    o1, h1, l1 = t.dense_attn_entropy(qp, k, v, wl.sm_scale, entropy=True, lse=True)
    o1n = t.tile_major_unpermute(o1, F, H, W, th, tw)
    o2, h2, l2 = t.dense_attn_entropy_natural(q, k, v, F, H, W, wl.sm_scale, entropy=True, lse=True, tile_h=th,
                                              tile_w=tw)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1n), _bits(o2)), "dense o"
    assert torch.equal(h1, h2), "entropy"
    assert torch.equal(l1, l2), "lse"
    # entropy off: the kernel without the entropy sums
    o3, _, _ = t.dense_attn_entropy(qp, k, v, wl.sm_scale, entropy=False)
    o4, _, _ = t.dense_attn_entropy_natural(q, k, v, F, H, W, wl.sm_scale, entropy=False, tile_h=th, tile_w=tw)
    assert torch.equal(_bits(t.tile_major_unpermute(o3, F, H, W, th, tw)), _bits(o4)), "dense o (no entropy)"

    # sparse: the permuted chain
    cnt, idx, _ = t.build_block_mask(h2, F, H, W, wl.tau, wl.gamma, wl.block_q, wl.block_k, wl.vote_threshold,
                                     th, tw)
    s1, sl1 = t.block_sparse_attn(qp, kp, vp, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    s2, sl2 = t.block_sparse_attn_natural(q, k, v, cnt, idx, F, H, W, wl.block_q, wl.block_k, wl.sm_scale, lse=True,
                                          tile_h=th, tile_w=tw)
    torch.cuda.synchronize()
    assert torch.equal(_bits(t.tile_major_unpermute(s1, F, H, W, th, tw)), _bits(s2)), "sparse o"
    assert torch.equal(sl1, sl2), "sparse lse"
    say("  block density %.3f" % float(cnt.float().sum().item() / (cnt.shape[0] * cnt.shape[1] * idx.shape[2])))
    return o2, h2, l2


@pytest.mark.parametrize("F,H,W,tile", [
    (4, 16, 16, (8, 8)),
    (3, 15, 20, (8, 8)),      # N = 900: ragged last q- and k-block; clipped tiles 7 x 8 and 7 x 4
    (2, 45, 80, (8, 8)),      # one 720p latent frame pair: 5-row edge tiles, k-blocks straddling tiles
    (5, 30, 52, (8, 8)),      # 480p-like rows: 4-wide edge tiles
    (3, 21, 24, (6, 12)),     # other tile shapes
    (2, 9, 28, (4, 4)),
    (1, 4, 8, (8, 8)),        # N = 32: one ragged tile
    (1, 1, 4, (8, 8)),        # N = 4: one run of four rows
])
def test_natural_equals_tile_major_calls(orc, F, H, W, tile):
    # bit for bit the tile-major calls; the dense outputs of every query of both heads against
    # the oracle
    t = tra()
    wl = _wl(300 + F + H + W, F, H, W, tile)
    say("natural order", F, H, W, tile)
    qc, kc, vc = qkv_inputs(wl)
    o, ent, lse = _compare(t, wl, qc.to(device()), kc.to(device()), vc.to(device()))
    _check_dense_natural(orc, wl, (qc, kc, vc), o, ent, lse)


def _check_dense_natural(orc, wl, qkv, o, ent, lse):
    """natural-order dense outputs (o natural, entropy and lse tile-major) of every query of
    every head against the oracle"""
    o, ent, lse = o.float().cpu().numpy(), ent.cpu().numpy(), lse.cpu().numpy()
    perm = orc.tile_major_order(wl.F, wl.H, wl.W, wl.tile_h, wl.tile_w)
    worst = [0.0, 0.0, 0.0]
    for h in range(wl.outer):
        ro, rH, rL = orc.attention(*(np64(x[h]) for x in qkv), wl.sm_scale)
        err, _ = check_output(o[h], ro, "bf16")                    # natural order
        e_ent = float(np.max(np.abs(ent[h] - rH[perm])))           # tile-major order
        e_lse = float(np.max(np.abs(lse[h] - rL[perm])))
        assert e_ent <= 1e-3, "head %d entropy err %.3g" % (h, e_ent)
        assert e_lse <= LSE_TOL, "head %d lse err %.3g" % (h, e_lse)
        worst = [max(worst[0], err), max(worst[1], e_ent), max(worst[2], e_lse)]
    say("  natural dense vs oracle: max-abs out %.3g, entropy %.3g, lse %.3g" % tuple(worst))


def test_natural_sparse_every_list_length():
    # lists of 0 to 16 k-blocks, with and without the ragged last k-block (N = 1000): the natural
    # kernel switches from copies between its products to copies at the step's start at a
    # different step for every length; it equals the permuted chain bit for bit throughout
    torch = torch_mod()
    t = tra()
    wl = _wl(321, 1, 25, 40)
    say("natural order, every list length")
    q, k, v = (x.to(device()) for x in qkv_inputs(wl))
    rng = np.random.default_rng(17)
    cnt = np.zeros((wl.outer, wl.nqb), dtype=np.int32)
    idx = np.full((wl.outer, wl.nqb, wl.nkb), -5, dtype=np.int32)
    for h in range(wl.outer):
        for qb in range(wl.nqb):
            n = (2 * qb + h) % (wl.nkb + 1)
            chosen = set(rng.choice(wl.nkb, size=n, replace=False).tolist())
            if n and (qb + h) % 2 and wl.nkb - 1 not in chosen:
                chosen.discard(min(chosen))
                chosen.add(wl.nkb - 1)
            cnt[h, qb] = n
            idx[h, qb, :n] = sorted(chosen)
    assert set(range(wl.nkb)) <= set(cnt.ravel().tolist())
    cnt_d, idx_d = torch.from_numpy(cnt).to(device()), torch.from_numpy(idx).to(device())
    F, H, W = wl.F, wl.H, wl.W
    qp, kp, vp = (t.tile_major_permute(x, F, H, W) for x in (q, k, v))
    s1, l1 = t.block_sparse_attn(qp, kp, vp, cnt_d, idx_d, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    s2, l2 = t.block_sparse_attn_natural(q, k, v, cnt_d, idx_d, F, H, W, wl.block_q, wl.block_k, wl.sm_scale,
                                         lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(t.tile_major_unpermute(s1, F, H, W)), _bits(s2)), "sparse o"
    assert torch.equal(l1, l2), "sparse lse"


@pytest.mark.parametrize("F,H,W,tile,vote", [
    (4, 16, 16, (8, 8), 1),
    (3, 15, 20, (8, 8), 2),   # ragged blocks, clipped tiles
    (2, 45, 80, (8, 8), 1),   # odd number of q-blocks
    (3, 21, 24, (6, 12), 1),
    (1, 4, 8, (8, 8), 1),     # one ragged q-block
])
def test_natural_fused_warmup(orc, F, H, W, tile, vote):
    torch = torch_mod()
    t = tra()
    wl = _wl(400 + F + H + W, F, H, W, tile)
    say("natural fused warm-up", F, H, W, tile, vote)
    qkv = qkv_inputs(wl)
    q, k, v = (x.to(device()) for x in qkv)
    th, tw = tile
    qp = t.tile_major_permute(q, F, H, W, th, tw)
    args = (F, H, W, wl.tau, wl.gamma, wl.sm_scale, wl.block_q, wl.block_k, vote, th, tw)
    # bit for bit the tile-major fused call on permuted q with k, v as given (keys in natural order)
    o1, h1, l1, c1, i1, m1 = t.dense_attn_entropy_mask(qp, k, v, *args, lse=True, want_mask=True)
    o2, h2, l2, c2, i2, m2 = t.dense_attn_entropy_mask_natural(q, k, v, *args, lse=True, want_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(t.tile_major_unpermute(o1, F, H, W, th, tw)), _bits(o2)), "o"
    assert torch.equal(h1, h2) and torch.equal(l1, l2), "entropy / lse"
    assert torch.equal(c1, c2) and torch.equal(m1, m2), "counts / mask"
    c = c1.cpu().numpy()
    a, b = i1.cpu().numpy(), i2.cpu().numpy()
    for hh in range(c.shape[0]):
        for qb in range(c.shape[1]):
            assert np.array_equal(a[hh, qb, :c[hh, qb]], b[hh, qb, :c[hh, qb]]), (hh, qb)
    # every query and q-block of both heads against the oracle
    check_warmup_against_oracle(orc, wl, qkv, (o2, h2, l2, c2, i2, m2), range(wl.outer), np.arange(wl.nqb), vote,
                                natural=True)


@pytest.mark.parametrize("wid", [3, 4])
def test_natural_fused_full_size(orc, wid):
    # natural-order fused warm-up over every head and q-block; seeded q-blocks (the ragged last one
    # included) of two seeded heads against the oracle
    t = tra()
    wl = workloads.get(wid)
    say("natural fused warm-up at full size", wl.name)
    qkv = qkv_inputs(wl)
    q, k, v = (x.to(device()) for x in qkv)
    t.mask_prepare(wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k)
    t.natural_prepare(wl.F, wl.H, wl.W)
    out = t.dense_attn_entropy_mask_natural(q, k, v, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.sm_scale, wl.block_q,
                                            wl.block_k, wl.vote_threshold, lse=True, want_mask=True)
    torch_mod().cuda.synchronize()
    del q, k, v
    blocks, _ = sample_rows(60 + wid, wl.N, wl.block_q, 3)
    heads = synth.uniform_ints(70 + wid, 2, 0, wl.outer)
    check_warmup_against_oracle(orc, wl, qkv, out, heads, blocks, wl.vote_threshold, natural=True)


def _lists_from_mask(mask):
    """mask [outer][nqb][nkb] -> int32 kv_count, kv_index (ascending, padded with -3)"""
    outer, nqb, nkb = mask.shape
    cnt = mask.sum(axis=2).astype(np.int32)
    idx = np.full((outer, nqb, nkb), -3, dtype=np.int32)
    for o in range(outer):
        for qb in range(nqb):
            nz = np.nonzero(mask[o, qb])[0]
            idx[o, qb, :len(nz)] = nz
    return cnt, idx


def _check_sparse_natural(orc, wl, qkv, o_nat, L, mask, heads, blocks):
    """natural-order sparse output rows of the q-blocks `blocks` vs the oracle's masked attention
    (tile-major positions, mask [nqb][nkb] per head), mapped to natural order"""
    torch = torch_mod()
    perm = orc.tile_major_order(wl.F, wl.H, wl.W, wl.tile_h, wl.tile_w)
    rows = rows_of_blocks(blocks, wl.N, wl.block_q)
    worst = 0.0
    for h in heads:
        qp, kp, vp = (orc.permute(np64(x[h]), perm) for x in qkv)
        ro, _, rL = orc.attention(qp, kp, vp, wl.sm_scale, rows=rows, block_mask=mask[h], bq=wl.block_q,
                                  bk=wl.block_k)
        sel = torch.from_numpy(perm[rows].astype(np.int64)).to(o_nat.device)
        err, _ = check_output(o_nat[h].index_select(0, sel).float().cpu().numpy(), ro, wl.dtype)
        r = torch.from_numpy(rows.astype(np.int64)).to(o_nat.device)
        e_lse = float(np.max(np.abs(L[h].index_select(0, r).cpu().numpy() - rL)))
        assert e_lse <= LSE_TOL, "head %d lse err %.3g" % (h, e_lse)
        worst = max(worst, err)
    say("  natural sparse vs oracle: max-abs %.3g" % worst)


@pytest.mark.parametrize("F,H,W,tile,tau", [
    (3, 15, 20, (8, 8), 0.03),    # ragged last q- and k-block; clipped 7 x 8 and 7 x 4 tiles
    (3, 21, 24, (6, 12), 0.02),
    (2, 9, 28, (4, 4), 0.05),
    (5, 12, 20, (8, 8), 0.002),   # short lists
    (1, 4, 8, (8, 8), 0.03),      # N = 32: one ragged tile
])
def test_natural_sparse_against_oracle(orc, F, H, W, tile, tau):
    # block lists from the oracle's mask of seeded entropies; every query of both heads
    torch = torch_mod()
    t = tra()
    wl = _wl(500 + F + H + W, F, H, W, tile, tau=tau)
    say("natural sparse vs oracle", F, H, W, tile, tau)
    qkv = qkv_inputs(wl)
    q, k, v = (x.to(device()) for x in qkv)
    ent = synth.entropy_like(600 + F + H, wl.outer, wl.N)
    mask = np.stack([orc.block_mask(ent[h], F, H, W, tau, wl.gamma, wl.block_q, wl.block_k, 1, tile[0],
                                    tile[1])[0] for h in range(wl.outer)])
    cnt, idx = _lists_from_mask(mask)
    o, L = t.block_sparse_attn_natural(q, k, v, torch.from_numpy(cnt).to(device()), torch.from_numpy(idx).to(device()),
                                       F, H, W, wl.block_q, wl.block_k, wl.sm_scale, lse=True, tile_h=tile[0],
                                       tile_w=tile[1])
    torch.cuda.synchronize()
    _check_sparse_natural(orc, wl, qkv, o, L, mask, range(wl.outer), np.arange(wl.nqb))


def test_natural_sparse_full_size_against_oracle(orc):
    # Wan2.1-14B shape: block lists from the GPU mask builder on seeded entropies; seeded q-blocks of
    # two seeded heads against the oracle's masked attention with its own mask rows of the same
    # entropies
    torch = torch_mod()
    t = tra()
    wl = workloads.get(3)
    say("natural sparse vs oracle at full size", wl.name)
    qkv = qkv_inputs(wl)
    q, k, v = (x.to(device()) for x in qkv)
    ent = synth.entropy_like(303, wl.outer, wl.N)
    cnt, idx, _ = t.build_block_mask(torch.from_numpy(ent).to(device()), wl.F, wl.H, wl.W, wl.tau, wl.gamma,
                                     wl.block_q, wl.block_k, wl.vote_threshold)
    t.natural_prepare(wl.F, wl.H, wl.W)
    o, L = t.block_sparse_attn_natural(q, k, v, cnt, idx, wl.F, wl.H, wl.W, wl.block_q, wl.block_k, wl.sm_scale,
                                       lse=True)
    torch.cuda.synchronize()
    del q, k, v
    blocks, _ = sample_rows(80, wl.N, wl.block_q, 3)
    heads = synth.uniform_ints(81, 2, 0, wl.outer)
    mask = np.zeros((wl.outer, wl.nqb, wl.nkb), dtype=np.uint8)
    for h in heads:
        mask[h][blocks], _ = orc.block_mask(ent[h], wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k,
                                            wl.vote_threshold, qblocks=blocks)
    _check_sparse_natural(orc, wl, qkv, o, L, mask, heads, blocks)


def test_natural_full_size_workload3():
    torch = torch_mod()
    t = tra()
    wl = workloads.get(3)
    say("natural order at full size", wl.name)
    q, k, v = (x.to(device()) for x in qkv_inputs(wl))
    F, H, W = wl.F, wl.H, wl.W
    qp = t.tile_major_permute(q, F, H, W)
    # dense: the tile-major call on permuted q and natural-order k, v
    o1, h1, _ = t.dense_attn_entropy(qp, k, v, wl.sm_scale, entropy=True)
    o1n = t.tile_major_unpermute(o1, F, H, W)
    d2, h2, _ = t.dense_attn_entropy_natural(q, k, v, F, H, W, wl.sm_scale, entropy=True)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2), "entropy at full size"
    assert torch.equal(_bits(o1n), _bits(d2)), "dense o at full size"
    del o1n, d2
    # sparse: the permuted chain
    kp, vp = (t.tile_major_permute(x, F, H, W) for x in (k, v))
    cnt, idx, _ = t.build_block_mask(h1, F, H, W, wl.tau, wl.gamma, wl.block_q, wl.block_k, wl.vote_threshold)
    s1, _ = t.block_sparse_attn(qp, kp, vp, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale, out=o1)
    del qp, kp, vp
    s1n = t.tile_major_unpermute(s1, F, H, W)
    del s1
    s2, _ = t.block_sparse_attn_natural(q, k, v, cnt, idx, F, H, W, wl.block_q, wl.block_k, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(_bits(s1n), _bits(s2)), "sparse o at full size"


def test_natural_rejects_unsupported():
    torch = torch_mod()
    t = tra()
    q = torch.zeros((1, 2 * 6 * 18, 128), dtype=torch.bfloat16, device=device())
    with pytest.raises(t.TraError) as ei:
        t.dense_attn_entropy_natural(q, q.clone(), q.clone(), 2, 6, 18)   # W = 18
    assert ei.value.code == 2
