"""GPU: the order of the block-sparse workgroups (tra_sparse_schedule; "Token Radius Attention for
Efficient Video Generation", section 4: 9-19% of the interactions kept with per-query budgets that
differ by orders of magnitude, hence rows of unequal work).

The schedule only moves work between workgroups: the scheduled calls equal the unscheduled ones bit
for bit (those are pinned to the oracle in test_gpu_attention.py and test_gpu_fp8.py).  The orders
themselves are checked against their definitions: a permutation of the rows; longest first by
kv_count with ties by row for short grids; for long grids the spatial band order dealt to the 8
XCDs in runs of 64.
"""
import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth, workloads
from gpu_util import device, qkv_inputs, say, small_workload, torch_mod, tra

pytestmark = pytest.mark.gpu

RUN = 64


def _band_reference(F, H, W, bq, outer, th=8, tw=8):
    """the documented band order, written out here: per head, q-blocks sorted by (row of tiles,
    frame, position along the row of tiles) of their centre token, then dealt to XCD b mod 8 in runs"""
    N = F * H * W
    nqb = -(-N // bq)
    keys = []
    for qb in range(nqb):
        p0 = min(qb * bq + bq // 2, N - 1)
        f, r = divmod(p0, H * W)
        keys.append((r // (th * W), f, r % (th * W), qb))
    band = [k[3] for k in sorted(keys)]
    total = outer * nqb
    full = (total // (8 * RUN)) * (8 * RUN)
    order = np.empty(total, dtype=np.int64)
    for b in range(total):
        if b < full:
            x, k = b & 7, b >> 3
            L = (k // RUN) * (8 * RUN) + x * RUN + (k % RUN)
        else:
            L = b
        o, r = divmod(L, nqb)
        order[b] = o * nqb + band[r]
    return order


def _compare_scheduled(t, wl, qp, kp, vp, cnt, idx, order):
    torch = torch_mod()
    o1, l1 = t.block_sparse_attn(qp, kp, vp, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    o2, l2 = t.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
    torch.cuda.synchronize()
    bits = (lambda x: x.view(torch.int16)) if qp.dtype == torch.bfloat16 else (lambda x: x)
    assert torch.equal(bits(o1), bits(o2)) and torch.equal(l1, l2), "scheduled call differs"


def test_schedule_longest_first_small_grid():
    # a few hundred rows: fewer than 2 waves of resident workgroups -> longest first
    torch = torch_mod()
    t = tra()
    wl = small_workload(800, 6, 30, 52, 128, "bf16", outer=3, tau=0.01)
    say("schedule longest first", wl.F, wl.H, wl.W)
    q, k, v = (t.tile_major_permute(x.to(device()), wl.F, wl.H, wl.W) for x in qkv_inputs(wl))
    ent = torch.from_numpy(synth.entropy_like(801, wl.outer, wl.N)).to(device())
    cnt, idx, _ = t.build_block_mask(ent, wl.F, wl.H, wl.W, wl.tau, wl.gamma)
    order = t.sparse_schedule(cnt, wl.F, wl.H, wl.W)
    torch.cuda.synchronize()
    c = cnt.cpu().numpy().ravel()
    ordv = order.cpu().numpy()
    assert np.array_equal(np.sort(ordv), np.arange(c.size))
    ref = np.lexsort((np.arange(c.size), -c))   # largest count first, ties by row
    assert np.array_equal(ordv, ref)
    _compare_scheduled(t, wl, q, k, v, cnt, idx, order)
    # fp32 kernel and 64-query blocks take the same orders
    wl64 = small_workload(802, 2, 9, 13, 128, "f32", bq=64, tau=0.05)
    q, k, v = (t.tile_major_permute(x.to(device()), wl64.F, wl64.H, wl64.W) for x in qkv_inputs(wl64))
    ent = torch.from_numpy(synth.entropy_like(803, wl64.outer, wl64.N)).to(device())
    cnt, idx, _ = t.build_block_mask(ent, wl64.F, wl64.H, wl64.W, wl64.tau, wl64.gamma, 64)
    order = t.sparse_schedule(cnt, wl64.F, wl64.H, wl64.W, block_q=64)
    _compare_scheduled(t, wl64, q, k, v, cnt, idx, order)


@pytest.mark.parametrize("wid", [3, 2])
def test_schedule_full_size(wid):
    # Wan2.1-14B (23,640 rows) and Wan2.1-1.3B (3,072 rows): both past 2 waves of resident workgroups,
    # the band order; with the GPU masks of the workload entropies, scheduled bf16 and fp8 calls equal
    # the unscheduled ones
    torch = torch_mod()
    t = tra()
    wl = workloads.get(wid)
    say("schedule full size", wl.name)
    q, k, v = qkv_inputs(wl)
    qp, kp, vp = (t.tile_major_permute(x.to(device()), wl.F, wl.H, wl.W) for x in (q, k, v))
    ent = torch.from_numpy(synth.entropy_like(810 + wid, wl.outer, wl.N)).to(device())
    cnt, idx, _ = t.build_block_mask(ent, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k)
    order = t.sparse_schedule(cnt, wl.F, wl.H, wl.W, wl.block_q, wl.block_k)
    torch.cuda.synchronize()
    ordv = order.cpu().numpy()
    total = wl.outer * wl.nqb
    assert np.array_equal(np.sort(ordv), np.arange(total))
    if total >= 2 * 512:
        assert np.array_equal(ordv, _band_reference(wl.F, wl.H, wl.W, wl.block_q, wl.outer))
    else:
        c = cnt.cpu().numpy().ravel()
        assert np.all(np.diff(c[ordv]) <= 0)
    _compare_scheduled(t, wl, qp, kp, vp, cnt, idx, order)
    q8, k8 = (t.tile_major_permute(x.to(device()).to(torch.float8_e4m3fn), wl.F, wl.H, wl.W) for x in (q, k))
    del qp, kp
    f1, m1 = t.block_sparse_attn_fp8(q8, k8, vp, cnt, idx, lse=True)
    f2, m2 = t.block_sparse_attn_fp8(q8, k8, vp, cnt, idx, lse=True, order=order)
    torch.cuda.synchronize()
    assert torch.equal(f1.view(torch.int16), f2.view(torch.int16)) and torch.equal(m1, m2), "scheduled fp8 differs"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_scheduled_out_of_contract_order(kind):
    # order entries outside [0, rows) are clamped into that range and a duplicated row runs twice:
    # every access stays inside the buffers, each row some entry names (after clamping) equals the
    # unscheduled call bit for bit, and rows no entry names keep what the output held before
    torch = torch_mod()
    t = tra()
    wl = small_workload(820, 3, 15, 20, 128, "bf16", outer=2, tau=0.05)
    say("out-of-contract order", kind, wl.F, wl.H, wl.W)
    q, k, v = (t.tile_major_permute(x.to(device()), wl.F, wl.H, wl.W) for x in qkv_inputs(wl))
    if kind == "fp8":
        q, k = q.to(torch.float8_e4m3fn), k.to(torch.float8_e4m3fn)
    ent = torch.from_numpy(synth.entropy_like(821, wl.outer, wl.N)).to(device())
    cnt, idx, _ = t.build_block_mask(ent, wl.F, wl.H, wl.W, wl.tau, wl.gamma)
    total = wl.outer * wl.nqb
    ordv = np.arange(total, dtype=np.int32)
    ordv[0] = -7            # clamps to row 0 (still named)
    ordv[1] = total + 50    # clamps to the last row (the ragged q-block of the last head): row 1 unnamed
    ordv[3] = ordv[2]       # row 2 twice, row 3 unnamed
    named = set(np.clip(ordv, 0, total - 1).tolist())
    order = torch.from_numpy(ordv).to(device())
    o = torch.full_like(v, float("nan"))
    lse = torch.full((wl.outer, wl.N), float("nan"), dtype=torch.float32, device=device())
    if kind == "fp8":
        ref, ref_l = t.block_sparse_attn_fp8(q, k, v, cnt, idx, lse=True)
        t.block_sparse_attn_fp8(q, k, v, cnt, idx, lse=True, order=order, out=o, lse_out=lse)
    else:
        ref, ref_l = t.block_sparse_attn(q, k, v, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale, lse=True)
        t.block_sparse_attn_scheduled(q, k, v, cnt, idx, order, wl.block_q, wl.block_k, wl.sm_scale, lse=True,
                                      out=o, lse_out=lse)
    torch.cuda.synchronize()
    for row in range(total):
        hd, qb = divmod(row, wl.nqb)
        sl = slice(qb * wl.block_q, min(wl.N, (qb + 1) * wl.block_q))
        if row in named:
            assert torch.equal(o[hd, sl].view(torch.int16), ref[hd, sl].view(torch.int16)), "row %d" % row
            assert torch.equal(lse[hd, sl], ref_l[hd, sl]), "lse row %d" % row
        else:
            assert bool(torch.isnan(o[hd, sl].float()).all()) and bool(torch.isnan(lse[hd, sl]).all()), \
                "unnamed row %d written" % row
