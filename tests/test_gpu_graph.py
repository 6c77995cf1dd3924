"""GPU: the step recorded into a HIP graph.  After the prepare calls no entry point allocates,
copies between host and device or clears memory, so the whole warm-up step (permute q, k, v;
dense attention with entropy; mask; schedule; scheduled block-sparse attention; unpermute) and
the natural-order reuse step and the natural-order warm-up (one call) can be captured once and
replayed, and so can the variants (the 1D-distance mask, its schedule, the fp8-score sparse
call).  Every replay, on fresh inputs copied
into the captured buffers (eager work and a synchronisation before each), equals the same calls
made eagerly on those inputs bit for bit."""
import math

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth
from gpu_util import device, say, torch_mod, tra

pytestmark = pytest.mark.gpu

F, H, W, OUTER, D = 6, 24, 40, 4, 128
TAU, GAMMA = 0.04, 0.5
SEEDS = (401, 402, 403)


def _inputs(torch, seed):
    q, k, v = synth.qkv(seed, OUTER, F, H, W, D, 0.25, 8.0)
    return [torch.from_numpy(x).to(torch.bfloat16).to(device()) for x in (q, k, v)]


def _lists_equal(torch, cnt_a, idx_a, cnt_b, idx_b):
    # kv_index rows are defined up to their counts; the rest of a row is left as it was
    if not torch.equal(cnt_a, cnt_b):
        return False
    valid = torch.arange(idx_a.shape[2], device=idx_a.device)[None, None, :] < cnt_a[:, :, None]
    return torch.equal(torch.where(valid, idx_a, 0), torch.where(valid, idx_b, 0))


def test_step_graph_replays_equal_eager():
    torch = torch_mod()
    t = tra()
    dev = device()
    N = F * H * W
    nqb, nkb = -(-N // 128), -(-N // 64)
    sc = 1.0 / math.sqrt(D)
    t.mask_prepare(F, H, W, TAU, GAMMA)
    t.natural_prepare(F, H, W)

    q, k, v = (torch.empty((OUTER, N, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    qp, kp, vp, od, osp, o, onat = (torch.empty_like(q) for _ in range(7))
    ent = torch.empty((OUTER, N), dtype=torch.float32, device=dev)
    cnt = torch.empty((OUTER, nqb), dtype=torch.int32, device=dev)
    idx = torch.zeros((OUTER, nqb, nkb), dtype=torch.int32, device=dev)
    order = torch.empty((OUTER * nqb,), dtype=torch.int32, device=dev)

    def warmup_step():
        for src, dst in ((q, qp), (k, kp), (v, vp)):
            t.tile_major_permute(src, F, H, W, out=dst)
        t.dense_attn_entropy(qp, kp, vp, sc, entropy=True, out=od, ent_out=ent)
        t.build_block_mask(ent, F, H, W, TAU, GAMMA, kv_count=cnt, kv_index=idx)
        t.sparse_schedule(cnt, F, H, W, out=order)
        t.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, sm_scale=sc, out=osp)
        t.tile_major_unpermute(osp, F, H, W, out=o)

    def reuse_step():
        t.block_sparse_attn_natural(q, k, v, cnt, idx, F, H, W, sm_scale=sc, out=onat)

    # the warm-up step as one call on natural-order tensors (its own outputs)
    onw = torch.empty_like(q)
    entn = torch.empty_like(ent)
    cntn = torch.empty_like(cnt)
    idxn = torch.zeros_like(idx)

    def natural_warmup():
        t.dense_attn_entropy_mask_natural(q, k, v, F, H, W, TAU, GAMMA, sc, out=onw, ent_out=entn, kv_count=cntn,
                                          kv_index=idxn)

    def load(seed):
        for dst, src in zip((q, k, v), _inputs(torch, seed)):
            dst.copy_(src)
        torch.cuda.synchronize()

    # eager references (these calls also load every kernel before the capture)
    ref = {}
    for seed in SEEDS:
        load(seed)
        warmup_step()
        reuse_step()
        natural_warmup()
        torch.cuda.synchronize()
        ref[seed] = [x.clone() for x in (od, ent, cnt, idx, order, o, onat, onw, entn, cntn, idxn)]
    say("eager density %.3f" % float(ref[SEEDS[0]][2].float().mean() / nkb))

    g_warm, g_reuse, g_nat = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        warmup_step()
    with torch.cuda.graph(g_reuse):
        reuse_step()
    with torch.cuda.graph(g_nat):
        natural_warmup()
    torch.cuda.synchronize()

    for rep, seed in enumerate(SEEDS + SEEDS[::-1]):
        say("replay", rep, "seed", seed)
        load(seed)
        g_warm.replay()
        torch.cuda.synchronize()
        r_od, r_ent, r_cnt, r_idx, r_order, r_o, r_onat, r_onw, r_entn, r_cntn, r_idxn = ref[seed]
        assert torch.equal(od, r_od), "dense o, replay %d" % rep
        assert torch.equal(ent, r_ent), "entropy, replay %d" % rep
        assert _lists_equal(torch, cnt, idx, r_cnt, r_idx), "block lists, replay %d" % rep
        assert torch.equal(order, r_order), "schedule, replay %d" % rep
        assert torch.equal(o, r_o), "sparse o, replay %d" % rep
        # the reuse step replays on the lists the warm-up replay just wrote
        g_reuse.replay()
        torch.cuda.synchronize()
        assert torch.equal(onat, r_onat), "natural-order reuse o, replay %d" % rep
        g_nat.replay()
        torch.cuda.synchronize()
        assert torch.equal(onw, r_onw), "natural-order warm-up o, replay %d" % rep
        assert torch.equal(entn, r_entn), "natural-order warm-up entropy, replay %d" % rep
        assert _lists_equal(torch, cntn, idxn, r_cntn, r_idxn), "natural-order warm-up lists, replay %d" % rep
    assert np.isfinite(o.float().cpu().numpy()).all()


def test_variants_graph_replays_equal_eager():
    # the 1D-distance mask, its schedule and the fp8-score sparse call taking that order, recorded
    # after tra_mask_prepare_1d: every replay on fresh q, k, v and entropies equals the eager calls
    torch = torch_mod()
    t = tra()
    dev = device()
    N = F * H * W
    nqb, nkb = -(-N // 128), -(-N // 64)
    sc = 1.0 / math.sqrt(D)
    t.mask_prepare_1d(F, H, W, TAU)

    q8, k8 = (torch.empty((OUTER, N, D), dtype=torch.float8_e4m3fn, device=dev) for _ in range(2))
    v = torch.empty((OUTER, N, D), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(v)
    ent = torch.empty((OUTER, N), dtype=torch.float32, device=dev)
    lse = torch.empty((OUTER, N), dtype=torch.float32, device=dev)
    cnt = torch.empty((OUTER, nqb), dtype=torch.int32, device=dev)
    idx = torch.zeros((OUTER, nqb, nkb), dtype=torch.int32, device=dev)
    order = torch.empty((OUTER * nqb,), dtype=torch.int32, device=dev)

    def step():
        t.build_block_mask_1d(ent, F, H, W, TAU, kv_count=cnt, kv_index=idx)
        t.sparse_schedule(cnt, F, H, W, out=order)
        t.block_sparse_attn_fp8(q8, k8, v, cnt, idx, sm_scale=sc, lse=True, order=order, out=o, lse_out=lse)

    def load(seed):
        qn, kn, vn = _inputs(torch, seed)
        for dst, src in ((q8, qn), (k8, kn), (v, vn)):
            dst.copy_(t.tile_major_permute(src, F, H, W).to(dst.dtype))
        ent.copy_(torch.from_numpy(synth.entropy_like(seed, OUTER, N)).to(dev))
        torch.cuda.synchronize()

    ref = {}
    for seed in SEEDS:
        load(seed)
        step()
        torch.cuda.synchronize()
        ref[seed] = [x.clone() for x in (cnt, idx, order, o, lse)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep, seed in enumerate(SEEDS[::-1] + SEEDS):
        say("variant replay", rep, "seed", seed)
        load(seed)
        g.replay()
        torch.cuda.synchronize()
        r_cnt, r_idx, r_order, r_o, r_lse = ref[seed]
        assert _lists_equal(torch, cnt, idx, r_cnt, r_idx), "1D lists, replay %d" % rep
        assert torch.equal(order, r_order), "schedule, replay %d" % rep
        assert torch.equal(o.view(torch.int16), r_o.view(torch.int16)), "fp8 sparse o, replay %d" % rep
        assert torch.equal(lse, r_lse), "fp8 sparse lse, replay %d" % rep
