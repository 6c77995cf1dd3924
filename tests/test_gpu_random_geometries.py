"""GPU parity over seeded random geometries ("Token Radius Attention for Efficient Video
Generation", section 2: the TRA pipeline from entropies to the block-sparse mask to block-sparse
attention).  Each case draws a grid (2-6 frames of 8-40 tokens a side, at most 4,000 tokens;
ragged q-blocks and k-blocks), a tile shape, block_q, a vote threshold, tau and gamma from its
seed, then checks on two heads:
  - the mask, counts and index lists bit for bit against the oracle's brute force;
  - the scheduled block-sparse attention (bf16 or fp32, D = 64 or 128, drawn per case) on those
    lists against the oracle's masked attention on every query, at the dtype's tolerances, with
    lse within 1e-3.
The same for the fused warm-up, tile-major and natural order (o, entropy, lse within the
tolerances; mask rows between the oracle's masks from its own entropies moved by the entropy
tolerance), and the natural-order sparse call on the natural fused call's lists (bit for
bit the tile-major call; against the oracle, under the oracle's mask, on every q-block whose
mask row the oracle fixes).  And the 1D-distance mask (bit for bit against the oracle) with
the fp8-score sparse call in the schedule's order on its block_q = 128 lists (against the
oracle on the decoded fp8 and bf16 inputs, lse within 1e-3 plus the fp8 instruction's
score-error bound).  And dense attention + entropy (bf16 or fp32, D = 64 or 128) on every query
against the oracle, with the permutation and its inverse bit for bit.  The fixed
cases elsewhere pin the shapes that matter most; these reach combinations nobody chose by
hand."""
import math

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import (LSE_TOL, check_output, check_warmup_against_oracle, device, fp8_group_truncation_bound, np64,
                      qkv_inputs, rows_of_blocks, say, torch_mod, tra)

pytestmark = pytest.mark.gpu

D = 128
OUTER = 2


def _case(seed):
    rng = np.random.default_rng(seed)
    while True:  # 2-6 frames of 8-40 tokens a side, at most 4,000 tokens (the fp64 oracle stays fast)
        F = int(rng.integers(2, 7))
        H = int(rng.integers(8, 41))
        W = int(rng.integers(8, 41))
        if F * H * W <= 4000:
            break
    th = int(rng.integers(1, 17))
    tw = int(rng.integers(1, 17))
    bq = int(rng.choice([64, 128]))
    vote = int(rng.integers(1, 4))
    tau = float(np.float32(10.0 ** rng.uniform(-3.0, -1.0)))
    gamma = float(np.float32(rng.uniform(0.0, 1.5)))
    return F, H, W, th, tw, bq, vote, tau, gamma


@pytest.mark.parametrize("seed", range(1000, 1016))
def test_random_geometry_mask_and_sparse(orc, seed):
    torch = torch_mod()
    t = tra()
    dev = device()
    F, H, W, th, tw, bq, vote, tau, gamma = _case(seed)
    N = F * H * W
    # the attention's head size and dtype from a stream of their own (the geometry stays as drawn)
    rng = np.random.default_rng(seed + 7919)
    Dh = int(rng.choice([64, 128]))
    dt = str(rng.choice(["bf16", "f32"]))
    say("random geometry", seed, (F, H, W), "tile", (th, tw), "bq", bq, "vote", vote, "tau %.4g gamma %.3g" % (tau, gamma),
        "D", Dh, dt)

    # mask: every q-block of both heads, bit for bit
    ent = synth.entropy_like(seed, OUTER, N)
    cnt, idx, msk = t.build_block_mask(torch.from_numpy(ent).to(dev), F, H, W, tau, gamma, bq, 64, vote, th, tw,
                                       want_mask=True)
    torch.cuda.synchronize()
    cnt_h, idx_h, msk_h = cnt.cpu().numpy(), idx.cpu().numpy(), msk.cpu().numpy()
    refs = []
    for h in range(OUTER):
        ref, _ = orc.block_mask(ent[h], F, H, W, tau, gamma, bq, 64, vote, th, tw)
        assert np.array_equal(msk_h[h], ref), "head %d mask" % h
        rc, lists = orc.mask_to_lists(ref)
        assert np.array_equal(cnt_h[h], rc), "head %d counts" % h
        for qb in range(ref.shape[0]):
            assert np.array_equal(idx_h[h, qb, :rc[qb]], lists[qb]), "head %d q-block %d list" % (h, qb)
        refs.append(ref)
    say("  density %.3f" % float(msk_h.mean()))

    # scheduled sparse attention on the GPU lists against the oracle's masked attention
    q, k, v = synth.qkv(seed, OUTER, F, H, W, Dh)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    qc, kc, vc = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
    qp, kp, vp = (t.tile_major_permute(x.to(dev), F, H, W, th, tw) for x in (qc, kc, vc))
    order = t.sparse_schedule(cnt, F, H, W, bq, 64, th, tw)
    scale = 1.0 / math.sqrt(Dh)
    o, L = t.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, bq, 64, scale, lse=True)
    torch.cuda.synchronize()
    o_h, L_h = o.float().cpu().numpy(), L.cpu().numpy()
    perm = orc.tile_major_order(F, H, W, th, tw)
    worst = 0.0
    for h in range(OUTER):
        # the oracle takes the same (rounded) inputs the GPU read, in fp64
        qh, kh, vh = (orc.permute(np64(x[h]), perm) for x in (qc, kc, vc))
        ro, _, rL = orc.attention(qh, kh, vh, scale, block_mask=refs[h], bq=bq, bk=64)
        err, _ = check_output(o_h[h], ro, dt)
        worst = max(worst, err)
        e_lse = float(np.max(np.abs(L_h[h] - rL)))
        assert e_lse <= LSE_TOL, "head %d lse err %.3g" % (h, e_lse)
    say("  sparse max-abs %.3g" % worst)


@pytest.mark.parametrize("seed", range(1100, 1108))
def test_random_geometry_fused_warmup(orc, seed):
    # the fused warm-up (tile-major on even seeds; natural order on odd ones, then the natural-order
    # sparse call on its lists) against the oracle: o, entropy and lse within the tolerances, the
    # mask rows between the oracle's masks from its own entropies moved by the entropy tolerance
    torch = torch_mod()
    t = tra()
    dev = device()
    F, H, W, th, tw, _, vote, tau, gamma = _case(seed)
    natural = seed % 2 == 1
    if natural:  # the natural-order calls move rows in runs of four
        W = min(40, -(-W // 4) * 4)
        tw = min(16, -(-tw // 4) * 4)
    wl = workloads.Workload(seed, "random-%dx%dx%d" % (F, H, W), 1, OUTER, D, "bf16", F, H, W, 128, 64, tau, gamma,
                            vote, th, tw)
    say("random fused warm-up", seed, (F, H, W), "tile", (th, tw), "vote", vote, "tau %.4g gamma %.3g" % (tau, gamma),
        "natural" if natural else "tile-major")
    q, k, v = qkv_inputs(wl)
    if natural:
        qd, kd, vd = (x.to(dev) for x in (q, k, v))
        out = t.dense_attn_entropy_mask_natural(qd, kd, vd, F, H, W, tau, gamma, wl.sm_scale, 128, 64, vote, th, tw,
                                                entropy=True, lse=True, want_mask=True)
    else:
        qd, kd, vd = (t.tile_major_permute(x.to(dev), F, H, W, th, tw) for x in (q, k, v))
        out = t.dense_attn_entropy_mask(qd, kd, vd, F, H, W, tau, gamma, wl.sm_scale, 128, 64, vote, th, tw,
                                        entropy=True, lse=True, want_mask=True)
    torch.cuda.synchronize()
    bounds = check_warmup_against_oracle(orc, wl, (q, k, v), out, range(OUTER), np.arange(wl.nqb), vote, natural)
    if natural:
        # the reuse step on those lists, natural order in and out: bit for bit the tile-major sparse
        # call on the permuted tensors, and, on the q-blocks whose mask rows the oracle's own entropies
        # fix, within the bf16 tolerances of the oracle's masked attention under the oracle's mask
        _, _, _, cnt, idx, _ = out
        o, L = t.block_sparse_attn_natural(qd, kd, vd, cnt, idx, F, H, W, 128, 64, wl.sm_scale, lse=True, tile_h=th,
                                           tile_w=tw)
        qp, kp, vp = (t.tile_major_permute(x, F, H, W, th, tw) for x in (qd, kd, vd))
        o2, L2 = t.block_sparse_attn(qp, kp, vp, cnt, idx, 128, 64, wl.sm_scale, lse=True)
        o2 = t.tile_major_unpermute(o2, F, H, W, th, tw)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "natural vs tile-major sparse o"
        assert torch.equal(L, L2), "natural vs tile-major sparse lse"
        perm = orc.tile_major_order(F, H, W, th, tw)
        o_h, L_h = o.float().cpu().numpy(), L.cpu().numpy()
        for h, (lo, hi) in zip(range(OUTER), bounds):
            # the q-blocks whose mask rows the oracle's entropies fix exactly (all but a rare row
            # with an entry the entropy tolerance leaves open)
            fixed = [qb for qb in range(wl.nqb) if np.array_equal(lo[qb], hi[qb])]
            if not fixed:
                continue
            rows = rows_of_blocks(fixed, wl.N, 128)
            qh, kh, vh = (orc.permute(np64(x[h]), perm) for x in (q, k, v))
            ro, _, rL = orc.attention(qh, kh, vh, wl.sm_scale, rows=rows, block_mask=lo, bq=128, bk=64)
            err, _ = check_output(o_h[h][perm][rows], ro, "bf16")
            e_lse = float(np.max(np.abs(L_h[h][rows] - rL)))
            assert e_lse <= LSE_TOL, "head %d natural sparse lse err %.3g" % (h, e_lse)
            say("  head %d natural sparse, %d of %d q-blocks fixed: max-abs %.3g" % (h, len(fixed), wl.nqb, err))


@pytest.mark.parametrize("seed", range(1200, 1208))
def test_random_geometry_mask1d_and_fp8(orc, seed):
    torch = torch_mod()
    t = tra()
    dev = device()
    F, H, W, th, tw, bq, vote, tau, _ = _case(seed)
    N = F * H * W
    say("random 1D mask + fp8", seed, (F, H, W), "tile", (th, tw), "bq", bq, "vote", vote, "tau %.4g" % tau)
    ent = synth.entropy_like(seed, OUTER, N)
    ent_d = torch.from_numpy(ent).to(dev)
    lists = {}
    for b in sorted({bq, 128}):
        cnt, idx, msk = t.build_block_mask_1d(ent_d, F, H, W, tau, b, 64, vote, th, tw, want_mask=True)
        torch.cuda.synchronize()
        cnt_h, idx_h, msk_h = cnt.cpu().numpy(), idx.cpu().numpy(), msk.cpu().numpy()
        refs = []
        for h in range(OUTER):
            ref, _ = orc.block_mask_1d(ent[h], F, H, W, tau, b, 64, vote, th, tw)
            assert np.array_equal(msk_h[h], ref), "block_q %d head %d mask" % (b, h)
            rc, rl = orc.mask_to_lists(ref)
            assert np.array_equal(cnt_h[h], rc), "block_q %d head %d counts" % (b, h)
            for qb in range(ref.shape[0]):
                assert np.array_equal(idx_h[h, qb, :rc[qb]], rl[qb]), "block_q %d head %d q-block %d" % (b, h, qb)
            refs.append(ref)
        lists[b] = (cnt, idx, refs)
        say("  block_q %d density %.3f" % (b, float(msk_h.mean())))

    # fp8 scores on the block_q = 128 lists, in the schedule's order
    cnt, idx, refs = lists[128]
    q, k, v = synth.qkv(seed, OUTER, F, H, W, D)
    q8, k8 = (torch.from_numpy(x).to(torch.float8_e4m3fn) for x in (q, k))
    vb = torch.from_numpy(v).to(torch.bfloat16)
    qp, kp, vp = (t.tile_major_permute(x.to(dev), F, H, W, th, tw) for x in (q8, k8, vb))
    order = t.sparse_schedule(cnt, F, H, W, 128, 64, th, tw)
    scale = 1.0 / math.sqrt(D)
    o, L = t.block_sparse_attn_fp8(qp, kp, vp, cnt, idx, sm_scale=scale, lse=True, order=order)
    torch.cuda.synchronize()
    o_h, L_h = o.float().cpu().numpy(), L.cpu().numpy().astype(np.float64)
    perm = orc.tile_major_order(F, H, W, th, tw)
    rows = np.arange(N, dtype=np.int32)
    worst, worst_lse = 0.0, 0.0
    for h in range(OUTER):
        # the oracle on the values the fp8 and bf16 inputs decode to, in fp64
        qh, kh, vh = (orc.permute(np64(x[h]), perm) for x in (q8, k8, vb))
        ro, _, rL = orc.attention(qh, kh, vh, scale, block_mask=refs[h], bq=128, bk=64)
        err, _ = check_output(o_h[h], ro, "bf16")
        bound = fp8_group_truncation_bound(qh, kh, rows, scale)
        fin = np.isfinite(rL)
        d = np.abs(L_h[h] - rL)[fin]
        assert np.all(d <= LSE_TOL + bound[fin]), "head %d fp8 lse beyond the bound" % h
        worst, worst_lse = max(worst, err), max(worst_lse, float(d.max()) if d.size else 0.0)
    say("  fp8 sparse max-abs %.3g, lse %.3g" % (worst, worst_lse))


@pytest.mark.parametrize("seed", range(1300, 1308))
def test_random_geometry_dense_and_permutation(orc, seed):
    # dense attention + entropy (bf16 or fp32, D = 64 or 128) on the tile-major permuted inputs of a
    # random geometry and tile shape: o, entropy and lse of every query of both heads against the
    # oracle's fp64 attention; the permutation and its inverse bit for bit against the oracle's
    # enumerated order
    torch = torch_mod()
    t = tra()
    dev = device()
    F, H, W, th, tw, _, _, _, _ = _case(seed)
    N = F * H * W
    rng = np.random.default_rng(seed + 7919)
    Dh = int(rng.choice([64, 128]))
    dt = str(rng.choice(["bf16", "f32"]))
    say("random dense", seed, (F, H, W), "tile", (th, tw), "D", Dh, dt)
    q, k, v = synth.qkv(seed, OUTER, F, H, W, Dh)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    qc, kc, vc = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
    perm = orc.tile_major_order(F, H, W, th, tw)
    qp, kp, vp = (t.tile_major_permute(x.to(dev), F, H, W, th, tw) for x in (qc, kc, vc))
    back = t.tile_major_unpermute(qp, F, H, W, th, tw)
    torch.cuda.synchronize()
    bits = (lambda x: x.view(torch.int16)) if dt == "bf16" else (lambda x: x.view(torch.int32))
    assert torch.equal(bits(qp.cpu()), bits(qc[:, torch.from_numpy(perm)])), "permutation"
    assert torch.equal(bits(back.cpu()), bits(qc)), "round trip"
    scale = 1.0 / math.sqrt(Dh)
    o, Hh, L = t.dense_attn_entropy(qp, kp, vp, scale, entropy=True, lse=True)
    torch.cuda.synchronize()
    o_h, H_h, L_h = o.float().cpu().numpy(), Hh.cpu().numpy(), L.cpu().numpy()
    worst = [0.0, 0.0, 0.0]
    for h in range(OUTER):
        qh, kh, vh = (orc.permute(np64(x[h]), perm) for x in (qc, kc, vc))
        ro, rH, rL = orc.attention(qh, kh, vh, scale)
        err, _ = check_output(o_h[h], ro, dt)
        e_ent = float(np.max(np.abs(H_h[h] - rH)))
        e_lse = float(np.max(np.abs(L_h[h] - rL)))
        assert e_ent <= 1e-3 and e_lse <= LSE_TOL, "head %d entropy %.3g lse %.3g" % (h, e_ent, e_lse)
        worst = [max(worst[0], err), max(worst[1], e_ent), max(worst[2], e_lse)]
    say("  dense vs oracle: max-abs out %.3g, entropy %.3g, lse %.3g" % tuple(worst))
