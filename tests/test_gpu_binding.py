"""GPU: the Python binding checks every caller-supplied buffer (shape, dtype, device,
contiguity) before it passes a pointer to the C ABI, so no kernel writes past a buffer the
caller sized wrongly."""
import pytest

from gpu_util import device, say, torch_mod, tra

pytestmark = pytest.mark.gpu


def test_binding_checks_every_buffer():
    torch = torch_mod()
    t = tra()
    dev = device()
    say("binding buffer checks")
    outer, F, H, W, D = 2, 2, 8, 16, 128
    N = F * H * W
    nqb, nkb = N // 128, N // 64
    q = torch.randn((outer, N, D), device=dev).to(torch.bfloat16)
    bf, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8

    def e(shape, dtype):
        return torch.empty(shape, dtype=dtype, device=dev)
    bad_dense = [dict(out=e((outer, N - 1, D), bf)), dict(out=e((outer, N, D), f32)),
                 dict(out=e((outer, D, N), bf).transpose(1, 2)), dict(ent_out=e((outer, N + 1), f32)),
                 dict(ent_out=e((outer, N), bf)), dict(lse_out=e((outer, N), f32)[:, :-1], lse=True)]
    for kw in bad_dense:
        with pytest.raises(ValueError):
            t.dense_attn_entropy(q, q, q, **kw)
    cnt, idx, _ = t.build_block_mask(torch.zeros((outer, N), device=dev), F, H, W, 0.05, 0.5)
    for kw in (dict(kv_count=e((outer, nqb + 1), i32)), dict(kv_index=e((outer, nqb, nkb), torch.int64)),
               dict(block_mask=e((outer, nqb, nkb - 1), u8))):
        with pytest.raises(ValueError):
            t.build_block_mask(torch.zeros((outer, N), device=dev), F, H, W, 0.05, 0.5, **kw)
    for args, kw in (((cnt[:, :-1].contiguous(), idx), {}), ((cnt, idx.to(torch.int64)), {}),
                     ((cnt, idx), dict(out=e((outer, N, D), f32))), ((cnt, idx), dict(lse=True, lse_out=e((1, N), f32)))):
        with pytest.raises(ValueError):
            t.block_sparse_attn(q, q, q, *args, **kw)
    with pytest.raises(ValueError):
        t.dense_attn_entropy_mask(q, q, q, F, H, W, 0.05, 0.5, kv_index=e((outer, nqb, nkb + 1), i32))
    with pytest.raises(ValueError):
        t.tile_major_permute(q, F, H, W, out=e((outer, N, D), f32))
    # correctly shaped buffers are accepted and written
    o, Hh, _ = t.dense_attn_entropy(q, q, q, out=e((outer, N, D), bf), ent_out=e((outer, N), f32))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(Hh).all())
