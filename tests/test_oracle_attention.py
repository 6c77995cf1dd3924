"""Pins of the oracle's attention and entropy against closed forms and invariants.

Attention and entropy follow "Token Radius Attention for Efficient Video Generation"
(section 1: dense 3D self-attention; section 2, Insight I and pipeline step 1: the
per-query attention entropy of the dense warm-up).  None of these tests recomputes the
oracle's formula: each checks a value that mathematics fixes independently.
"""
import math

import numpy as np
import pytest


def _rng(seed):
    return np.random.default_rng(seed)


def test_uniform_logits_give_ln_n(orc):
    # q = 0 makes every logit equal: p = 1/N, H = ln N, o = mean(v), lse = ln N
    N, D = 300, 16
    r = _rng(1)
    q = np.zeros((N, D))
    k = r.standard_normal((N, D))
    v = r.standard_normal((N, D))
    o, H, lse = orc.attention(q, k, v)
    assert np.allclose(H, math.log(N), atol=1e-12)
    assert np.allclose(lse, math.log(N), atol=1e-12)
    assert np.allclose(o, v.mean(axis=0)[None, :], atol=1e-12)


def test_one_hot_gives_zero_entropy(orc):
    # orthonormal keys, query along key 3 with a logit gap of 800: every other weight
    # underflows to exactly 0 in fp64, so H = 0 and o = v_3
    N = D = 32
    k = np.eye(N)
    q = np.zeros((N, D))
    q[:, 3] = 800.0
    v = _rng(2).standard_normal((N, D))
    o, H, _ = orc.attention(q, k, v, scale=1.0)
    assert np.all(H == 0.0)
    assert np.allclose(o, v[3][None, :], atol=0)


@pytest.mark.parametrize("delta", [0.0, 0.3, 1.0, 2.5, 7.0, 20.0])
def test_two_keys_binary_entropy(orc, delta):
    # two keys with logits 0 and delta: softmax is the logistic split, and the entropy
    # is the binary entropy h(p) = -p ln p - (1-p) ln(1-p), p = 1 / (1 + e^delta)
    D = 4
    k = np.array([[0.0, 0, 0, 0], [1.0, 0, 0, 0]])
    q = np.array([[delta, 0, 0, 0]])
    qq = np.repeat(q, 2, axis=0)
    v = np.array([[1.0, 0, 0, 0], [0.0, 1.0, 0, 0]])
    o, H, lse = orc.attention(qq, k, v, scale=1.0, rows=[0])
    p = 1.0 / (1.0 + math.exp(delta))
    hb = -(p * math.log(p) + (1 - p) * math.log(1 - p))
    assert abs(H[0] - hb) < 1e-13
    assert abs(o[0, 0] - p) < 1e-13 and abs(o[0, 1] - (1 - p)) < 1e-13
    assert abs(lse[0] - math.log(1 + math.exp(delta))) < 1e-12


@pytest.mark.parametrize("m", [2, 3, 5])
def test_duplicated_keys_add_ln_m(orc, m):
    # Merging identical keys (FAST-AR summary, Lemma 5.1: identical keys merged with a
    # group-size logit shift are exact), read backwards: duplicating every (k, v) pair m
    # times leaves o unchanged and raises every entropy and lse by exactly ln m.
    N, D = 40, 8
    r = _rng(3)
    q, k, v = (r.standard_normal((N, D)) * 2 for _ in range(3))
    o1, H1, l1 = orc.attention(q, k, v)
    kk, vv = np.tile(k, (m, 1)), np.tile(v, (m, 1))
    qq = np.tile(q, (m, 1))
    o2, H2, l2 = orc.attention(qq, kk, vv, rows=np.arange(N))
    assert np.allclose(o2, o1, atol=1e-12)
    assert np.allclose(H2, H1 + math.log(m), atol=1e-12)
    assert np.allclose(l2, l1 + math.log(m), atol=1e-12)


def test_entropy_bounds_and_key_permutation(orc):
    N, D = 200, 16
    r = _rng(4)
    q = r.standard_normal((N, D)) * r.uniform(0.1, 6, size=(N, 1))
    k, v = r.standard_normal((N, D)), r.standard_normal((N, D))
    o, H, lse = orc.attention(q, k, v)
    assert np.all(H >= -1e-12) and np.all(H <= math.log(N) + 1e-12)
    sigma = r.permutation(N)
    o2, H2, lse2 = orc.attention(q, k[sigma], v[sigma])
    assert np.allclose(o2, o, atol=1e-12) and np.allclose(H2, H, atol=1e-12)
    assert np.allclose(lse2, lse, atol=1e-12)


def test_default_scale_is_inverse_sqrt_d(orc):
    N, D = 50, 64
    r = _rng(5)
    q, k, v = (r.standard_normal((N, D)) for _ in range(3))
    a = orc.attention(q, k, v)
    # scaling q by 1/sqrt(D) with unit scale must give the same result
    b = orc.attention(q / math.sqrt(D), k, v, scale=1.0)
    for x, y in zip(a, b):
        assert np.allclose(x, y, atol=1e-12)


def test_query_and_key_roles_not_swapped(orc):
    # a single strong key among many: only the query aligned with it concentrates;
    # swapping the roles of q and k would change which rows concentrate.
    N, D = 16, 16
    k = np.zeros((N, D))
    k[5, 0] = 50.0
    q = np.zeros((N, D))
    q[2, 0] = 1.0
    v = np.eye(N, D)
    o, H, _ = orc.attention(q, k, v, scale=1.0)
    assert H[2] < 1e-15 and abs(o[2, 5] - 1.0) < 1e-15
    for i in range(N):
        if i != 2:
            assert abs(H[i] - math.log(N)) < 1e-12


def test_all_ones_block_mask_equals_dense(orc):
    N, D, bq, bk = 150, 8, 64, 32
    r = _rng(6)
    q, k, v = (r.standard_normal((N, D)) for _ in range(3))
    mask = np.ones((-(-N // bq), -(-N // bk)), dtype=np.uint8)
    a = orc.attention(q, k, v)
    b = orc.attention(q, k, v, block_mask=mask, bq=bq, bk=bk)
    for x, y in zip(a, b):
        assert np.allclose(x, y, atol=1e-13)


def test_block_mask_equals_attention_on_the_retained_keys(orc):
    # a row sees exactly the tokens of its q-block's retained k-blocks (ragged last block)
    N, D, bq, bk = 150, 8, 64, 32
    r = _rng(7)
    q, k, v = (r.standard_normal((N, D)) for _ in range(3))
    nqb, nkb = -(-N // bq), -(-N // bk)
    mask = (r.uniform(size=(nqb, nkb)) < 0.4).astype(np.uint8)
    mask[:, 4] = 1  # the ragged last k-block (keys 128..149) everywhere
    o, H, lse = orc.attention(q, k, v, block_mask=mask, bq=bq, bk=bk)
    for i in range(N):
        keys = np.concatenate([np.arange(kb * bk, min(N, kb * bk + bk)) for kb in range(nkb) if mask[i // bq, kb]])
        sub = np.concatenate([q[i:i + 1], q[:len(keys) - 1]]) if len(keys) > 1 else q[i:i + 1]
        o2, H2, l2 = orc.attention(sub, k[keys], v[keys], rows=[0], scale=1.0 / math.sqrt(D))
        assert np.allclose(o[i], o2[0], atol=1e-13)
        assert abs(H[i] - H2[0]) < 1e-13 and abs(lse[i] - l2[0]) < 1e-13


def test_online_entropy_recurrence_equals_two_pass(orc):
    # The GPU accumulates the entropy in one pass in base 2: running max m, l = sum 2^(x-m),
    # t = sum 2^(x-m) (x-m); on a max change m -> m': a = 2^(m-m'), t <- a (t + (m - m') l),
    # l <- a l; finally H = ln2 (log2 l - t / l).  Here in fp64 over key tiles of 64,
    # also with the max kept stale until it grows by more than 8 (the lazy rescale).
    N, D = 1000, 32
    r = _rng(8)
    q = r.standard_normal((N, D)) * r.uniform(0.1, 8, size=(N, 1))
    k, v = r.standard_normal((N, D)), r.standard_normal((N, D))
    _, H, lse = orc.attention(q, k, v)
    x_all = (q @ k.T) / math.sqrt(D) / math.log(2.0)
    for lazy in (0.0, 8.0):
        for i in range(0, N, 97):
            m, l, t = -np.inf, 0.0, 0.0
            for j0 in range(0, N, 64):
                x = x_all[i, j0:j0 + 64]
                mt = max(m, x.max())
                if mt > m + lazy:
                    a = 0.0 if m == -np.inf else 2.0 ** (m - mt)
                    t = a * (t + ((m - mt) * l if l > 0 else 0.0))
                    l = a * l
                    m = mt
                e = 2.0 ** (x - m)
                l += e.sum()
                t += (e * (x - m)).sum()
            h = math.log(2.0) * (math.log2(l) - t / l)
            assert abs(h - H[i]) < 1e-10
            assert abs(math.log(2.0) * (m + math.log2(l)) - lse[i]) < 1e-10
