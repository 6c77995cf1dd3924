"""GPU: the fused warm-up pass (dense attention + entropy with the mask builder as its
epilogue, two q-blocks' rows per workgroup; "Token Radius Attention for Efficient Video
Generation", section 2, TRA pipeline steps 1-3) equals the two separate calls bit for bit.

The separate calls are pinned to the oracle elsewhere: tra_dense_attn_entropy in
test_gpu_attention.py (outputs, entropy and lse within tolerance), tra_build_block_mask in
test_gpu_mask.py (bit-exact masks from entropies the oracle also sees).  Here the fused
mask is compared with tra_build_block_mask applied to the fused call's own entropies, and
its o, entropy and lse with tra_dense_attn_entropy's: no oracle value comes from the GPU.
"""
import numpy as np
import pytest

from entropy_adaptive_sparse_amd import workloads
from gpu_util import device, qkv_inputs, say, small_workload, torch_mod, tra

pytestmark = pytest.mark.gpu


def _tile_major(t, wl):
    torch = torch_mod()
    q, k, v = qkv_inputs(wl)
    return tuple(t.tile_major_permute(x.to(device()), wl.F, wl.H, wl.W) for x in (q, k, v))


def _compare(t, wl, q, k, v, vote):
    torch = torch_mod()
    o1, h1, l1, c1, i1, m1 = t.dense_attn_entropy_mask(q, k, v, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.sm_scale,
                                                       wl.block_q, wl.block_k, vote, entropy=True, lse=True,
                                                       want_mask=True)
    o2, h2, l2 = t.dense_attn_entropy(q, k, v, wl.sm_scale, entropy=True, lse=True)
    c2, i2, m2 = t.build_block_mask(h1, wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k, vote,
                                    want_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "o"
    assert torch.equal(h1, h2), "entropy"
    assert torch.equal(l1, l2), "lse"
    assert torch.equal(c1, c2), "kv_count"
    assert torch.equal(m1, m2), "block mask"
    c = c1.cpu().numpy()
    a, b = i1.cpu().numpy(), i2.cpu().numpy()
    for h in range(c.shape[0]):
        for qb in range(c.shape[1]):
            assert np.array_equal(a[h, qb, :c[h, qb]], b[h, qb, :c[h, qb]]), (h, qb)
    return float(m1.float().mean().item())


@pytest.mark.parametrize("F,H,W,tau,gamma,vote", [
    (4, 16, 16, 0.03, 0.5, 1),
    (3, 15, 17, 0.02, 0.0, 2),       # ragged blocks and tiles, frames straddled by q-blocks
    (12, 5, 7, 0.05, 0.3, 1),        # several frames per q-block; more than 4 rectangles per k-block
    (40, 2, 3, 0.3, 0.1, 1),         # 6-token frames, 40 frames: thresholds in two LDS buffers
    (2, 45, 80, 0.03, 0.5, 3),
    (6, 30, 52, 0.001, 0.5, 1),
    (1, 8, 12, 0.05, 0.5, 1),        # one ragged q-block: the workgroup's second half has no row
    (2, 8, 8, 0.05, 0.5, 2),         # exactly one q-block
    (3, 7, 9, 0.05, 0.5, 1),         # N = 189: two q-blocks, the second ragged
])
def test_fused_equals_separate(F, H, W, tau, gamma, vote):
    t = tra()
    wl = small_workload(200 + F + H + W, F, H, W, 128, "bf16", tau=tau, gamma=gamma, vote=vote)
    say("fused warm-up", F, H, W, tau, gamma, vote)
    q, k, v = _tile_major(t, wl)
    dens = _compare(t, wl, q, k, v, vote)
    say("  block density", dens)


@pytest.mark.parametrize("wid", [3, 4])  # 4: 33 frames, thresholds in both split buffers
def test_fused_full_size(wid):
    t = tra()
    wl = workloads.get(wid)
    say("fused warm-up at full size", wl.name)
    q, k, v = _tile_major(t, wl)
    t.mask_prepare(wl.F, wl.H, wl.W, wl.tau, wl.gamma, wl.block_q, wl.block_k)
    dens = _compare(t, wl, q, k, v, wl.vote_threshold)
    say("  block density", dens)


def test_fused_rejects_unsupported():
    torch = torch_mod()
    t = tra()
    q = torch.zeros((1, 4 * 16 * 16, 64), dtype=torch.bfloat16, device=device())
    with pytest.raises(t.TraError) as ei:
        t.dense_attn_entropy_mask(q, q.clone(), q.clone(), 4, 16, 16, 0.03, 0.5)
    assert ei.value.code == 2
