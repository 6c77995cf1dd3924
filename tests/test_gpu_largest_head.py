"""GPU: block-sparse attention at the largest head the sparse calls accept ("Token Radius
Attention for Efficient Video Generation", section 2, pipeline step 3: the block-sparse
backend).  The tile-major sparse kernels copy K and V tiles as buffer loads with 32-bit byte
offsets inside one head, so a head's K (and V) must stay below 2^31 bytes.

Two heads of N = 2047 x 4097 = 8,386,559 tokens at D = 128: one head's bf16 K is 2^31 - 524,544
bytes, and almost all of the second head lies past 2^31 bytes from the tensor's start (64-bit
head offsets, 32-bit offsets within the head).  The last k-block is ragged (63 rows) and so
is the last q-block (127 rows).  Every q-block's list holds its own two k-blocks, one seeded
k-block and the last three, so every q-block copies the tiles at the top of the head's offset
range, between its products and at the step start.  bf16 in the schedule's order, and fp8
scores, on sampled q-blocks of both heads against the oracle (the oracle sees each sampled
q-block's queries against exactly its retained keys, from the same seeded rows).  Then the
tile-major permutation of those tensors, on seeded rows bit for bit.
"""
import functools
import math

import numpy as np
import pytest

from entropy_adaptive_sparse_amd import synth
from gpu_util import LSE_TOL, check_output, device, fp8_group_truncation_bound, say, torch_mod, tra

pytestmark = pytest.mark.gpu

HH, WW = 2047, 4097
N = HH * WW
D = 128
OUTER = 2
SEED = 41
CHUNK = 1 << 18
BQ, BK = 128, 64
NQB, NKB = -(-N // BQ), -(-N // BK)


def _lists():
    """kv_count [NQB], kv_index rows [NQB][6] (ascending, padded with the row's last entry)"""
    rng = np.random.default_rng(SEED)
    extra = rng.integers(0, NKB, size=NQB)
    cnt = np.zeros(NQB, dtype=np.int32)
    idx = np.zeros((NQB, 6), dtype=np.int32)
    for qb in range(NQB):
        row = sorted({2 * qb, min(2 * qb + 1, NKB - 1), int(extra[qb]), NKB - 3, NKB - 2, NKB - 1})
        cnt[qb] = len(row)
        idx[qb, :len(row)] = row
        idx[qb, len(row):] = row[-1]
    return cnt, idx


@functools.lru_cache(maxsize=8)
def _chunk(which, c):
    return synth.normal_chunk(SEED, which, c, min(CHUNK, N - c * CHUNK), D)


def _rows(which, rows):
    """the generator's float32 values of `rows` (ascending) of tensor `which`"""
    out = np.empty((len(rows), D), dtype=np.float32)
    for c in np.unique(rows // CHUNK):
        sel = (rows // CHUNK) == c
        out[sel] = _chunk(int(which), int(c))[rows[sel] - c * CHUNK]
    return out


def _as(x, dt):
    torch = torch_mod()
    return torch.from_numpy(x).to(dt).float().numpy().astype(np.float64)


def test_sparse_largest_head(orc):
    torch = torch_mod()
    t = tra()
    dev = device()
    assert N * D * 2 < 2 ** 31 <= 2 * N * D * 2 and N % BK == 63 and N % BQ == 127
    say("largest head: %d heads of N = %d, D = %d (%d bytes per head's K)" % (OUTER, N, D, N * D * 2))

    # q, k, v (tensor 3 h + 0, 1, 2 of the generator): bf16, and fp8 for q and k
    q, k, v = (torch.empty((OUTER, N, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    q8, k8 = (torch.empty((OUTER, N, D), dtype=torch.float8_e4m3fn, device=dev) for _ in range(2))
    for h in range(OUTER):
        for j, (dst, dst8) in enumerate(((q, q8), (k, k8), (v, None))):
            for s, a in synth.normal_rows(SEED, 3 * h + j, N, D, chunk_rows=CHUNK):
                x = torch.from_numpy(a)
                dst[h, s:s + len(a)].copy_(x.to(torch.bfloat16))
                if dst8 is not None:
                    dst8[h, s:s + len(a)].copy_(x.to(torch.float8_e4m3fn))
        say("  head %d filled" % h)

    cnt_h, idx_h = _lists()
    cnt = torch.from_numpy(np.stack([cnt_h] * OUTER)).to(dev)
    idx = torch.zeros((OUTER, NQB, NKB), dtype=torch.int32, device=dev)
    idx[:, :, :6] = torch.from_numpy(idx_h).to(dev)[None]
    scale = 1.0 / math.sqrt(D)
    order = t.sparse_schedule(cnt, 1, HH, WW, BQ, BK, 1, 1)
    o, L = t.block_sparse_attn_scheduled(q, k, v, cnt, idx, order, BQ, BK, scale, lse=True)
    o8, L8 = t.block_sparse_attn_fp8(q8, k8, v, cnt, idx, sm_scale=scale, lse=True)
    torch.cuda.synchronize()
    say("  sparse calls done")
    del idx, order, q, k, q8, k8
    torch.cuda.empty_cache()

    blocks = [0, NQB // 2, NQB - 1] + [int(b) for b in synth.uniform_ints(SEED, 1, 1, NQB - 1)]
    worst = [0.0, 0.0]
    for h in range(OUTER):
        for qb in blocks:
            rows = np.arange(qb * BQ, min(N, qb * BQ + BQ))
            keys = np.concatenate([np.arange(b * BK, min(N, b * BK + BK)) for b in idx_h[qb, :cnt_h[qb]]])
            assert len(keys) >= len(rows)
            qf, kf, vf = _rows(3 * h, rows), _rows(3 * h + 1, keys), _rows(3 * h + 2, keys)
            r = torch.from_numpy(rows).to(dev)
            # the queries padded to the number of keys: dense attention of those rows over exactly
            # the retained keys is the masked attention of the q-block
            for kind, qdt, kdt, oo, LL in (("bf16", torch.bfloat16, torch.bfloat16, o, L),
                                           ("fp8", torch.float8_e4m3fn, torch.float8_e4m3fn, o8, L8)):
                qs = np.zeros((len(keys), D))
                qs[:len(rows)] = _as(qf, qdt)
                ks, vs = _as(kf, kdt), _as(vf, torch.bfloat16)
                ro, _, rL = orc.attention(qs, ks, vs, scale, rows=np.arange(len(rows), dtype=np.int32))
                err, _ = check_output(oo[h].index_select(0, r).float().cpu().numpy(), ro, "bf16")
                d = np.abs(LL[h].index_select(0, r).cpu().numpy().astype(np.float64) - rL)
                tol = LSE_TOL + (fp8_group_truncation_bound(qs, ks, np.arange(len(rows)), scale) if kind == "fp8" else 0.0)
                assert np.all(d <= tol), "head %d q-block %d %s lse err %.3g" % (h, qb, kind, float(d.max()))
                worst[kind == "fp8"] = max(worst[kind == "fp8"], err)
        say("  head %d: sampled q-blocks %s match the oracle" % (h, blocks))
    say("  max-abs bf16 %.3g, fp8 %.3g" % tuple(worst))
    del o, L, o8, L8, cnt
    torch.cuda.empty_cache()

    # the permutation at this size (8 x 8 tiles; W = 4097 leaves a clipped column of 1-wide
    # tiles): seeded tile-major rows of both heads, bit for bit the generator's rows at the
    # oracle's enumerated order
    y = t.tile_major_permute(v, 1, HH, WW)
    torch.cuda.synchronize()
    perm = orc.tile_major_order(1, HH, WW)
    pos = np.unique(np.concatenate([synth.uniform_ints(SEED + 1, 2000, 0, N), [0, N - 1]])).astype(np.int64)
    for h in range(OUTER):
        got = y[h].index_select(0, torch.from_numpy(pos).to(dev)).cpu()
        src = np.sort(perm[pos])
        want = torch.from_numpy(_rows(3 * h + 2, src)).to(torch.bfloat16)
        order_back = np.argsort(np.argsort(perm[pos]))
        assert torch.equal(got.view(torch.int16), want[torch.from_numpy(order_back)].view(torch.int16)), "head %d" % h
    say("  permutation: %d seeded rows of each head bit for bit" % len(pos))
    del y, v
    torch.cuda.empty_cache()
