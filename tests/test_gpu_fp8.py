"""GPU parity: block-sparse attention with fp8 (OCP E4M3) queries and keys and bf16 values
("Token Radius Attention for Efficient Video Generation", section 5: TRA is complementary to
quantization; pipeline step 3: the reused block-sparse mask).

The oracle runs fp64 attention on the values the fp8 bytes of q and k and the bf16 values of v
decode to, restricted to its own block mask.  Tolerances:
- outputs: the bf16 ones (relative L2 <= 1e-2, max-abs <= 3e-2).  The probabilities are rounded
  to bf16 for the PV product as in the bf16 kernel.
- lse: 1e-3 plus a per-row bound of the score error of the fp8 matrix instruction.  Each product
  of two E4M3 values is exact, but the instruction sums every aligned group of 8 products in a
  fixed-point format 13 bits below the exponent of the group's largest product, dropping the bits
  below (measured with single-instruction sums of 1 + 2^-e: 2^-13 kept, 2^-14 lost), and adds the
  group sums in fp32.  So a score is off by less than the sum over its 16 groups of
  7 * 2^(e_g - 13) * sm_scale, e_g the exponent of the group's largest |q_d k_d|.  The softmax
  cancels such a shift only up to its variation across keys, which the output tolerance covers;
  the lse carries it, bounded by the largest such sum over the row's keys.
"""
import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import (LSE_TOL, check_output, device, fp8_group_truncation_bound, np64, qkv_inputs, sample_rows,
                      say, small_workload, torch_mod, tra)

pytestmark = pytest.mark.gpu


def _inputs(wl):
    """natural-order CPU tensors: q, k fp8 (rounded once from the generator's fp32 values), v bf16"""
    torch = torch_mod()
    q, k, v = qkv_inputs(wl, dtype=torch.float32)
    return q.to(torch.float8_e4m3fn), k.to(torch.float8_e4m3fn), v.to(torch.bfloat16)


def _tile_major(t, wl, q, k, v):
    return tuple(t.tile_major_permute(x.to(device()), wl.F, wl.H, wl.W) for x in (q, k, v))


def _lists(mask):
    outer, nqb, nkb = mask.shape
    cnt = mask.sum(axis=2).astype(np.int32)
    idx = np.full((outer, nqb, nkb), -9, dtype=np.int32)
    for o in range(outer):
        for qb in range(nqb):
            nz = np.nonzero(mask[o, qb])[0]
            idx[o, qb, :len(nz)] = nz
    return cnt, idx


def _check(orc, wl, q, k, v, o, L, mask, heads, rows):
    """o, L: GPU results (tile-major); q, k, v: natural-order CPU tensors"""
    torch = torch_mod()
    perm = orc.tile_major_order(wl.F, wl.H, wl.W)
    r = torch.from_numpy(rows.astype(np.int64)).to(o.device)
    worst, worst_lse = 0.0, 0.0
    for h in heads:
        qp, kp, vp = (orc.permute(np64(x[h]), perm) for x in (q, k, v))
        ro, _, rL = orc.attention(qp, kp, vp, wl.sm_scale, rows=rows, block_mask=mask[h], bq=wl.block_q,
                                  bk=wl.block_k)
        err, _ = check_output(o[h].index_select(0, r).float().cpu().numpy(), ro, "bf16")
        d_lse = L[h].index_select(0, r).cpu().numpy().astype(np.float64) - rL
        bound = fp8_group_truncation_bound(qp, kp, rows, wl.sm_scale)
        fin = np.isfinite(rL)
        # two-sided: the direction the dropped bits of a negative product go is not measured
        assert np.all(np.abs(d_lse[fin]) <= LSE_TOL + bound[fin]), "head %d lse beyond the bound" % h
        worst = max(worst, err)
        worst_lse = max(worst_lse, float(np.max(np.abs(d_lse[fin]))) if fin.any() else 0.0)
    say("  fp8 sparse vs oracle: max-abs %.3g, lse %.3g" % (worst, worst_lse))


def test_fp8_rounding_is_ocp_e4m3():
    # the inputs the tests build: E4M3 with bias 7, max 448, 3 mantissa bits (the format the kernel
    # reads); checked on values whose encodings are known
    torch = torch_mod()
    x = torch.tensor([1.0, 448.0, 0.015625, 1.0625, 1.125, -2.5, 2.0 ** -9], dtype=torch.float32)
    b = x.to(torch.float8_e4m3fn).view(torch.uint8).tolist()
    assert b == [0x38, 0x7E, 0x08, 0x38, 0x39, 0xC2, 0x01]


@pytest.mark.parametrize("F,H,W,tau", [
    (3, 15, 17, 0.03),     # N = 765: ragged last q- and k-block
    (4, 16, 16, 1.0),      # every block retained: dense attention on fp8 scores
    (5, 12, 20, 0.002),    # short lists
    (2, 30, 52, 0.01),
])
def test_fp8_sparse_small_full(orc, F, H, W, tau):
    torch = torch_mod()
    t = tra()
    wl = small_workload(700 + F + H, F, H, W, 128, "bf16", tau=tau)
    say("fp8 sparse small", F, H, W, tau)
    q, k, v = _inputs(wl)
    ent = synth.entropy_like(710 + F, wl.outer, wl.N)
    mask = np.stack([orc.block_mask(ent[h], F, H, W, tau, wl.gamma, 128, 64, 1)[0] for h in range(wl.outer)])
    cnt, idx = _lists(mask)
    qp, kp, vp = _tile_major(t, wl, q, k, v)
    o, L = t.block_sparse_attn_fp8(qp, kp, vp, torch.from_numpy(cnt).to(device()), torch.from_numpy(idx).to(device()),
                                   lse=True, sm_scale=wl.sm_scale)
    torch.cuda.synchronize()
    _check(orc, wl, q, k, v, o, L, mask, range(wl.outer), np.arange(wl.N, dtype=np.int32))


def test_fp8_every_list_length(orc):
    # lists of 0 to 16 k-blocks, half of them ending with the ragged k-block (N = 1000): the step at
    # which the copies move from between the products to the step's start differs for every length
    torch = torch_mod()
    t = tra()
    wl = small_workload(720, 1, 25, 40, 128, "bf16")
    say("fp8 sparse list lengths")
    q, k, v = _inputs(wl)
    rng = np.random.default_rng(721)
    mask = np.zeros((wl.outer, wl.nqb, wl.nkb), dtype=np.uint8)
    for h in range(wl.outer):
        for qb in range(wl.nqb):
            n = (2 * qb + h) % (wl.nkb + 1)
            chosen = rng.choice(wl.nkb, size=n, replace=False)
            if n and (qb + h) % 2:
                chosen[0] = wl.nkb - 1
                chosen = np.unique(chosen)
                while len(chosen) < n:
                    chosen = np.unique(np.append(chosen, rng.integers(0, wl.nkb)))
            mask[h, qb, chosen] = 1
    cnt, idx = _lists(mask)
    qp, kp, vp = _tile_major(t, wl, q, k, v)
    o, L = t.block_sparse_attn_fp8(qp, kp, vp, torch.from_numpy(cnt).to(device()), torch.from_numpy(idx).to(device()),
                                   lse=True, sm_scale=wl.sm_scale)
    torch.cuda.synchronize()
    empty = cnt == 0
    rows = np.array([r for r in range(wl.N) if not empty[0, r // 128] and not empty[1, r // 128]], dtype=np.int32)
    _check(orc, wl, q, k, v, o, L, mask, range(wl.outer), rows)
    oc = o.float().cpu().numpy()
    for h in range(wl.outer):
        for qb in np.nonzero(empty[h])[0]:
            assert float(np.abs(oc[h, qb * 128:(qb + 1) * 128]).max()) == 0.0


@pytest.mark.parametrize("wid", [3, 4])
def test_fp8_full_size_sampled(orc, wid):
    # Wan2.1-14B and HunyuanVideo shapes: every head and q-block on the GPU with the GPU mask of
    # seeded entropies; seeded q-blocks (the ragged last one included) of two seeded heads against
    # the oracle
    torch = torch_mod()
    t = tra()
    wl = workloads.get(wid)
    say("fp8 sparse full size", wl.name)
    q, k, v = _inputs(wl)
    ent = synth.entropy_like(727 + wid, wl.outer, wl.N)
    cnt, idx, _ = t.build_block_mask(torch.from_numpy(ent).to(device()), wl.F, wl.H, wl.W, wl.tau, wl.gamma,
                                     wl.block_q, wl.block_k, wl.vote_threshold)
    qp, kp, vp = _tile_major(t, wl, q, k, v)
    o, L = t.block_sparse_attn_fp8(qp, kp, vp, cnt, idx, lse=True, sm_scale=wl.sm_scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    blocks, rows = sample_rows(728 + 3 * wid, wl.N, 128, 3)
    heads = synth.uniform_ints(729 + 3 * wid, 2, 0, wl.outer)
    mask = np.zeros((wl.outer, wl.nqb, wl.nkb), dtype=np.uint8)
    for h in heads:
        mask[h][blocks], _ = orc.block_mask(ent[h], wl.F, wl.H, wl.W, wl.tau, wl.gamma, 128, 64, 1, qblocks=blocks)
    _check(orc, wl, q, k, v, o, L, mask, heads, rows)


def test_fp8_invalid_lists_stay_inside():
    # out-of-contract lists (the ragged k-block early, duplicates, out-of-range values, counts above
    # nkb) are clamped: with NaN right after k and v in memory the output stays finite
    torch = torch_mod()
    t = tra()
    dev = device()
    wl = small_workload(740, 1, 25, 40, 128, "bf16")
    outer, N, D, nkb, nqb = wl.outer, wl.N, 128, wl.nkb, wl.nqb
    say("fp8 sparse invalid lists")
    q, k, v = _inputs(wl)
    kbig = torch.full((outer * N + 256, D), 0x7F, dtype=torch.uint8, device=dev)   # 0x7F: E4M3 NaN
    vbig = torch.full((outer * N + 256, D), float("nan"), dtype=torch.bfloat16, device=dev)
    kbig[:outer * N] = t.tile_major_permute(k.to(dev), wl.F, wl.H, wl.W).view(torch.uint8).reshape(outer * N, D)
    vbig[:outer * N] = t.tile_major_permute(v.to(dev), wl.F, wl.H, wl.W).reshape(outer * N, D)
    kd = kbig[:outer * N].view(torch.float8_e4m3fn).view(outer, N, D)
    vd = vbig[:outer * N].view(outer, N, D)
    qd = t.tile_major_permute(q.to(dev), wl.F, wl.H, wl.W)
    rng = np.random.default_rng(741)
    idx = rng.integers(0, nkb, size=(outer, nqb, nkb)).astype(np.int32)
    idx[:, :, 0] = nkb - 1
    idx[:, :, 2] = nkb - 1
    idx[:, :, 5] = -4
    idx[:, :, 6] = nkb + 7
    cnt = np.full((outer, nqb), nkb + 3, dtype=np.int32)
    o, L = t.block_sparse_attn_fp8(qd, kd, vd, torch.from_numpy(cnt).to(dev), torch.from_numpy(idx).to(dev), lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(L).all())
