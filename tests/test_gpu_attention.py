"""GPU parity: dense warm-up attention + entropy, and block-sparse attention, against
the fp64 oracle on the same (bf16- or fp32-valued) inputs ("Token Radius Attention
for Efficient Video Generation", section 1; TRA pipeline steps 1 and 3).

Tolerances: entropy <= 1e-3 nats absolute; outputs fp32 max-abs <= 1e-4, bf16
relative L2 <= 1e-2 and max-abs <= 3e-2; lse <= 1e-3 absolute.
"""
import math

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import (check_output, device, qkv_inputs, say, sample_rows, small_workload, torch_mod, tra)

pytestmark = pytest.mark.gpu

ENT_TOL = 1e-3
LSE_TOL = 1e-3


def _to_gpu_tile_major(t, wl, q, k, v):
    torch = torch_mod()
    dev = device()
    qp = t.tile_major_permute(q.to(dev), wl.F, wl.H, wl.W)
    kp = t.tile_major_permute(k.to(dev), wl.F, wl.H, wl.W)
    vp = t.tile_major_permute(v.to(dev), wl.F, wl.H, wl.W)
    return qp, kp, vp


def _np64(x):
    return x.float().numpy().astype(np.float64)


def _check_dense(orc, wl, q, k, v, o, H, L, heads, rows=None):
    """o, H, L: GPU results (tile-major, CPU numpy).  rows: tile-major positions to check."""
    perm = orc.tile_major_order(wl.F, wl.H, wl.W)
    worst = [0.0, 0.0, 0.0]
    for h in heads:
        rr = np.arange(wl.N, dtype=np.int32) if rows is None else rows
        nat = perm[rr].astype(np.int32)
        ro, rH, rL = orc.attention(_np64(q[h]), _np64(k[h]), _np64(v[h]), wl.sm_scale, rows=nat)
        err, rl = check_output(o[h][rr], ro, wl.dtype)
        e_ent = float(np.max(np.abs(H[h][rr] - rH)))
        e_lse = float(np.max(np.abs(L[h][rr] - rL)))
        assert e_ent <= ENT_TOL, "head %d entropy err %.3g" % (h, e_ent)
        assert e_lse <= LSE_TOL, "head %d lse err %.3g" % (h, e_lse)
        worst = [max(worst[0], err), max(worst[1], e_ent), max(worst[2], e_lse)]
    say("  max-abs out %.3g, entropy %.3g, lse %.3g" % tuple(worst))


def _run_dense(t, wl, q, k, v):
    torch = torch_mod()
    qp, kp, vp = _to_gpu_tile_major(t, wl, q, k, v)
    o, H, L = t.dense_attn_entropy(qp, kp, vp, wl.sm_scale, entropy=True, lse=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), H.cpu().numpy(), L.cpu().numpy()


def test_dense_tiny_fp32_full(orc):
    wl = workloads.get(1)
    t = tra()
    say("dense tiny fp32 full")
    q, k, v = qkv_inputs(wl)
    o, H, L = _run_dense(t, wl, q, k, v)
    _check_dense(orc, wl, q, k, v, o, H, L, heads=range(wl.outer))


@pytest.mark.parametrize("F,H,W,D,dtype", [
    (3, 15, 17, 128, "bf16"),   # N = 765: ragged q-block and k-block
    (4, 16, 16, 64, "bf16"),
    (2, 9, 13, 64, "f32"),      # N = 234
    (3, 15, 17, 128, "f32"),
    (1, 1, 1, 128, "bf16"),     # a single token
    (1, 8, 8, 128, "bf16"),     # exactly one tile
])
def test_dense_small_full(orc, F, H, W, D, dtype):
    wl = small_workload(50 + D, F, H, W, D, dtype)
    t = tra()
    say("dense small", F, H, W, D, dtype)
    q, k, v = qkv_inputs(wl)
    o, Hh, L = _run_dense(t, wl, q, k, v)
    _check_dense(orc, wl, q, k, v, o, Hh, L, heads=range(wl.outer))


def test_dense_uniform_and_one_hot_closed_forms():
    # q = 0: every row uniform, H = ln N exactly in theory; one-hot rows: H ~ 0
    torch = torch_mod()
    t = tra()
    dev = device()
    N, D = 1000, 128
    q = torch.zeros((1, N, D), dtype=torch.bfloat16, device=dev)
    k = torch.randn((1, N, D), device=dev).to(torch.bfloat16)
    v = torch.randn((1, N, D), device=dev).to(torch.bfloat16)
    o, H, L = t.dense_attn_entropy(q, k, v, entropy=True, lse=True)
    torch.cuda.synchronize()
    assert float((H - math.log(N)).abs().max()) < 1e-3
    assert float((L - math.log(N)).abs().max()) < 1e-3
    ref = v.float().mean(dim=1, keepdim=True)
    assert float((o.float() - ref).abs().max()) < 1e-2
    # one-hot: keys e_j * 64 and queries e_i * 64 (scale 1): logit gap 4096 -> p = delta
    kk = torch.zeros((1, 128, D), device=dev)
    kk[0, torch.arange(128), torch.arange(128)] = 64.0
    o2, H2, _ = t.dense_attn_entropy(kk.to(torch.bfloat16), kk.to(torch.bfloat16),
                                     torch.eye(128, device=dev)[None].to(torch.bfloat16), sm_scale=1.0)
    torch.cuda.synchronize()
    assert float(H2.abs().max()) < 1e-3
    assert float((o2.float()[0] - torch.eye(128, device=dev)).abs().max()) < 1e-2


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_dense_full_size_sampled(orc, wid):
    wl = workloads.get(wid)
    t = tra()
    say("dense full size workload", wid, wl.name)
    q, k, v = qkv_inputs(wl)
    o, H, L = _run_dense(t, wl, q, k, v)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(H))
    assert np.all(H >= -ENT_TOL) and np.all(H <= math.log(wl.N) + ENT_TOL)
    _, rows = sample_rows(wid, wl.N, 128, 3)
    heads = synth.uniform_ints(wid + 10, 2, 0, wl.outer)
    _check_dense(orc, wl, q, k, v, o, H, L, heads=heads, rows=rows)
    say("  entropy p10/p50/p90: %.2f %.2f %.2f (ln N %.2f)" % (*np.percentile(H, [10, 50, 90]), math.log(wl.N)))


# ------------------------------------------------------------------ block-sparse
def _lists_from_mask(mask):
    """mask [outer][nqb][nkb] -> int32 kv_count, kv_index (padded with -7 past the count)."""
    outer, nqb, nkb = mask.shape
    cnt = mask.sum(axis=2).astype(np.int32)
    idx = np.full((outer, nqb, nkb), -7, dtype=np.int32)
    for o in range(outer):
        for qb in range(nqb):
            nz = np.nonzero(mask[o, qb])[0]
            idx[o, qb, :len(nz)] = nz
    return cnt, idx


def _oracle_masks(orc, ent, wl, heads, qblocks=None):
    mask = np.zeros((wl.outer, wl.nqb, wl.nkb), dtype=np.uint8)
    for h in heads:
        m, _ = orc.block_mask(ent[h], wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k,
                              wl.vote_threshold, qblocks=qblocks)
        if qblocks is None:
            mask[h] = m
        else:
            mask[h][qblocks] = m
    return mask


def _check_sparse(orc, wl, q, k, v, o, L, mask, heads, rows):
    perm = orc.tile_major_order(wl.F, wl.H, wl.W)
    worst = 0.0
    for h in heads:
        qp, kp, vp = (orc.permute(_np64(x[h]), perm) for x in (q, k, v))
        ro, _, rL = orc.attention(qp, kp, vp, wl.sm_scale, rows=rows, block_mask=mask[h], bq=wl.block_q,
                                  bk=wl.block_k)
        err, _ = check_output(o[h][rows], ro, wl.dtype)
        e_lse = float(np.max(np.abs(L[h][rows] - rL)))
        assert e_lse <= LSE_TOL, "lse err %.3g" % e_lse
        worst = max(worst, err)
    say("  sparse max-abs %.3g" % worst)


def _run_sparse(t, wl, q, k, v, cnt, idx):
    torch = torch_mod()
    dev = device()
    qp, kp, vp = _to_gpu_tile_major(t, wl, q, k, v)
    o, L = t.block_sparse_attn(qp, kp, vp, torch.from_numpy(cnt).to(dev), torch.from_numpy(idx).to(dev),
                               wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), L.cpu().numpy()


@pytest.mark.parametrize("F,H,W,D,dtype,bq,tau", [
    (3, 15, 17, 128, "bf16", 128, 0.03),
    (3, 15, 17, 128, "bf16", 64, 0.03),
    (4, 16, 16, 64, "bf16", 64, 0.01),
    (4, 16, 16, 64, "f32", 64, 1.0),
    (2, 9, 13, 128, "f32", 128, 0.05),
    (5, 12, 20, 128, "bf16", 128, 0.002),
])
def test_sparse_small_full(orc, F, H, W, D, dtype, bq, tau):
    wl = small_workload(80 + D + bq, F, H, W, D, dtype, bq=bq, tau=tau)
    t = tra()
    say("sparse small", F, H, W, D, dtype, bq, tau)
    q, k, v = qkv_inputs(wl)
    ent = synth.entropy_like(F + H + W, wl.outer, wl.N)
    mask = _oracle_masks(orc, ent, wl, range(wl.outer))
    cnt, idx = _lists_from_mask(mask)
    o, L = _run_sparse(t, wl, q, k, v, cnt, idx)
    _check_sparse(orc, wl, q, k, v, o, L, mask, range(wl.outer), np.arange(wl.N, dtype=np.int32))
    # cross-step reuse: a new draw of q, k, v with the same mask
    q2, k2, v2 = qkv_inputs(small_workload(wl.wid + 1, F, H, W, D, dtype, bq=bq, tau=tau))
    o2, L2 = _run_sparse(t, wl, q2, k2, v2, cnt, idx)
    _check_sparse(orc, wl, q2, k2, v2, o2, L2, mask, [0], np.arange(wl.N, dtype=np.int32))


@pytest.mark.parametrize("D,dtype,bq", [(128, "bf16", 128), (128, "bf16", 64), (64, "bf16", 128)])
def test_sparse_every_list_length(orc, D, dtype, bq):
    # Lists of 0 to 16 k-blocks, with and without the ragged last k-block (N = 1000): the
    # kernel copies tiles between its products while both tiles of a step's copies are full and
    # exist (list position + 3 < length), and at the step's start for the last steps; every
    # length crosses that switch at a different step.
    wl = small_workload(140 + D + bq, 1, 25, 40, D, dtype, bq=bq)
    t = tra()
    say("sparse list lengths", D, dtype, bq)
    q, k, v = qkv_inputs(wl)
    rng = np.random.default_rng(11 + D + bq)
    mask = np.zeros((wl.outer, wl.nqb, wl.nkb), dtype=np.uint8)
    for h in range(wl.outer):
        for qb in range(wl.nqb):
            n = (2 * qb + h) % (wl.nkb + 1)
            chosen = rng.choice(wl.nkb, size=n, replace=False)
            if n and (qb + h) % 2:  # half of the lists end with the ragged k-block
                chosen[0] = wl.nkb - 1
                chosen = np.unique(chosen)
                while len(chosen) < n:
                    chosen = np.unique(np.append(chosen, rng.integers(0, wl.nkb)))
            mask[h, qb, chosen] = 1
    cnt, idx = _lists_from_mask(mask)
    assert set(range(wl.nkb)) <= set(cnt.ravel().tolist())  # lengths 0 .. nkb - 1 at least
    o, L = _run_sparse(t, wl, q, k, v, cnt, idx)
    empty = cnt == 0
    rows = np.array([r for r in range(wl.N) if not empty[0, r // wl.block_q] and not empty[1, r // wl.block_q]],
                    dtype=np.int32)
    _check_sparse(orc, wl, q, k, v, o, L, mask, range(wl.outer), rows)
    for h in range(wl.outer):
        for qb in np.nonzero(empty[h])[0]:
            r0, r1 = qb * wl.block_q, min(wl.N, (qb + 1) * wl.block_q)
            assert float(np.abs(o[h, r0:r1]).max()) == 0.0 and bool(np.isinf(L[h, r0:r1]).all())


def test_sparse_all_blocks_equals_dense_bitexact():
    torch = torch_mod()
    t = tra()
    dev = device()
    for (N, D) in ((2000, 128), (1500, 64)):
        say("sparse all blocks == dense", N, D)
        q, k, v = (torch.randn((2, N, D), device=dev).to(torch.bfloat16) for _ in range(3))
        o_d, _, L_d = t.dense_attn_entropy(q, k, v, entropy=False, lse=True)
        nqb, nkb = -(-N // 128), -(-N // 64)
        cnt = torch.full((2, nqb), nkb, dtype=torch.int32, device=dev)
        idx = torch.arange(nkb, dtype=torch.int32, device=dev).repeat(2, nqb, 1).contiguous()
        o_s, L_s = t.block_sparse_attn(q, k, v, cnt, idx, 128, 64, lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o_d.view(torch.int16), o_s.view(torch.int16))
        assert torch.equal(L_d, L_s)


def test_sparse_empty_row_and_determinism():
    torch = torch_mod()
    t = tra()
    dev = device()
    N, D = 700, 128
    q, k, v = (torch.randn((1, N, D), device=dev).to(torch.bfloat16) for _ in range(3))
    nqb, nkb = -(-N // 128), -(-N // 64)
    cnt = torch.full((1, nqb), 3, dtype=torch.int32, device=dev)
    cnt[0, 2] = 0
    idx = torch.zeros((1, nqb, nkb), dtype=torch.int32, device=dev)
    idx[0, :, :3] = torch.tensor([0, 4, nkb - 1], dtype=torch.int32, device=dev)
    o1, L1 = t.block_sparse_attn(q, k, v, cnt, idx, lse=True)
    o2, L2 = t.block_sparse_attn(q, k, v, cnt, idx, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(L1, L2)
    assert float(o1[0, 256:384].float().abs().max()) == 0.0
    assert bool(torch.isinf(L1[0, 256:384]).all())


@pytest.mark.parametrize("wid", [3, 4, 2, 5])
def test_sparse_full_size_sampled(orc, wid):
    # every head and q-block runs on the GPU with a GPU-built mask; the oracle checks seeded
    # q-blocks of seeded heads against its own mask rows from the same entropy array
    wl = workloads.get(wid)
    t = tra()
    torch = torch_mod()
    dev = device()
    say("sparse full size workload", wid, wl.name, "tau", wl.tau)
    q, k, v = qkv_inputs(wl)
    if wl.static_mask:  # the per-head constants the benchmark uses
        ent = np.repeat(np.asarray(wl.static_entropy, dtype=np.float32)[:, None], wl.N, axis=1)
    else:
        ent = synth.entropy_like(300 + wid, wl.outer, wl.N)
    cnt, idx, _ = t.build_block_mask(torch.from_numpy(ent).to(dev), wl.F, wl.H, wl.W, wl.tau, wl.gamma,
                                     wl.block_q, wl.block_k, wl.vote_threshold)
    qp, kp, vp = _to_gpu_tile_major(t, wl, q, k, v)
    o, L = t.block_sparse_attn(qp, kp, vp, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    L = L.cpu().numpy()
    assert np.all(np.isfinite(o))
    blocks, rows = sample_rows(wid + 20, wl.N, wl.block_q, 3)
    heads = synth.uniform_ints(wid + 30, 2, 0, wl.outer)
    mask = _oracle_masks(orc, ent, wl, heads, qblocks=blocks)
    _check_sparse(orc, wl, q, k, v, o, L, mask, heads, rows)


@pytest.mark.parametrize("dtype,slope", [("bf16", 2.0), ("f32", 2.0), ("bf16", -2.0)])
def test_rising_scores_force_max_moves(orc, dtype, slope):
    # scores grow (or fall) along the natural key order by ~0.2 nats per key (~13 nats per
    # 64 keys), so a rising max outgrows the running reference by more than the lazy
    # threshold (2^8) in almost every tile: the O / l / t rescale runs tile after tile (dense
    # with entropy, and sparse over every block), and the result must still match the
    # two-pass oracle
    torch = torch_mod()
    t = tra()
    F, H, W, D = 1, 16, 40, 128
    N = F * H * W
    wl = small_workload(300, F, H, W, D, dtype, outer=1)
    g = np.random.default_rng(7)
    q = np.zeros((1, N, D), dtype=np.float32)
    q[0, :, 0] = 4.0 + g.uniform(0.0, 1.0, N)
    q[0, :, 1:] = 0.1 * g.standard_normal((N, D - 1))
    k = 0.1 * g.standard_normal((1, N, D)).astype(np.float32)
    k[0, :, 0] = slope * np.arange(N) / 4.0
    v = g.standard_normal((1, N, D)).astype(np.float32)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    qt, kt, vt = (torch.from_numpy(x).to(dt) for x in (q, k, v))
    o, Hh, L = _run_dense(t, wl, qt, kt, vt)
    _check_dense(orc, wl, qt, kt, vt, o, Hh, L, heads=[0])
    dev = device()
    qp, kp, vp = _to_gpu_tile_major(t, wl, qt, kt, vt)
    nqb, nkb = -(-N // wl.block_q), -(-N // wl.block_k)
    cnt = torch.full((1, nqb), nkb, dtype=torch.int32, device=dev)
    idx = torch.arange(nkb, dtype=torch.int32, device=dev).repeat(1, nqb, 1).contiguous()
    os_, Ls = t.block_sparse_attn(qp, kp, vp, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    od, _, Ld = t.dense_attn_entropy(qp, kp, vp, wl.sm_scale, entropy=False, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(os_, od) and torch.equal(Ls, Ld)  # every block retained: the dense result, bit for bit


@pytest.mark.parametrize("dtype,natural", [("bf16", False), ("f32", False), ("bf16", True)])
def test_sparse_invalid_lists_stay_inside(orc, dtype, natural):
    # Lists that break the contract -- the ragged last k-block at positions 0-2 (and again later),
    # duplicates, negative and too-large entries, a count above nkb -- are clamped as the header
    # states: every access stays inside k and v.  k and v end where a buffer holding NaN rows
    # begins, so a row read past N that entered a softmax would turn the output into NaN.  The
    # q-blocks with valid lists in the same call still match the oracle.
    torch = torch_mod()
    t = tra()
    dev = device()
    F, H, W, D = 1, 25, 40, 128   # N = 1000: nkb = 16 with a ragged 40-row k-block, nqb = 8
    wl = small_workload(170, F, H, W, D, dtype)
    N, nkb, nqb, outer = wl.N, wl.nkb, wl.nqb, wl.outer
    say("sparse invalid lists", dtype, "natural" if natural else "tile-major")
    q, k, v = qkv_inputs(wl)
    tdt = q.dtype
    bufs = []
    for x in (k, v):
        big = torch.full((outer * N + 256, D), float("nan"), dtype=tdt, device=dev)
        big[:outer * N] = x.reshape(outer * N, D).to(dev)
        bufs.append(big)
    kd, vd = (b[:outer * N].view(outer, N, D) for b in bufs)
    qd = q.to(dev)
    rng = np.random.default_rng(171)
    cnt = np.zeros((outer, nqb), dtype=np.int32)
    idx = np.zeros((outer, nqb, nkb), dtype=np.int32)
    mask = np.zeros((outer, nqb, nkb), dtype=np.uint8)
    for h in range(outer):
        for qb in range(nqb):
            if qb < 4:  # invalid lists
                n = nkb
                row = rng.integers(0, nkb, size=n).astype(np.int32)
                row[qb % 3] = nkb - 1
                row[(qb + 5) % n] = nkb - 1
                row[7] = -3 - qb
                row[9] = nkb + 40 * qb
                cnt[h, qb] = n + 3 * qb  # above nkb for qb > 0: clamped to nkb
                idx[h, qb] = row
            else:       # valid lists, the ragged k-block last in half of them
                n = 5 + qb
                chosen = np.sort(rng.choice(nkb - 1, size=n - (qb % 2), replace=False))
                if qb % 2:
                    chosen = np.append(chosen, nkb - 1)
                cnt[h, qb] = len(chosen)
                idx[h, qb, :len(chosen)] = chosen
                mask[h, qb, chosen] = 1
    cd, id_ = torch.from_numpy(cnt).to(dev), torch.from_numpy(idx).to(dev)
    if natural:
        qn, kn, vn = qd, kd, vd
        o_nat, L = t.block_sparse_attn_natural(qn, kn, vn, cd, id_, F, H, W, wl.block_q, wl.block_k, wl.sm_scale,
                                               lse=True)
        o = t.tile_major_permute(o_nat, F, H, W)
    else:
        # tile-major copies whose k and v again end where the NaN rows begin
        for b, x in zip(bufs, (kd, vd)):
            b[:outer * N] = t.tile_major_permute(x.clone(), F, H, W).reshape(outer * N, D)
        qp = t.tile_major_permute(qd, F, H, W)
        o, L = t.block_sparse_attn(qp, kd, vd, cd, id_, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    L = L.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(L)), "a row past N reached the softmax"
    rows = np.arange(4 * wl.block_q, N, dtype=np.int32)
    _check_sparse(orc, wl, q, k, v, o, L, mask, range(outer), rows)
