"""Pins of the paged-attention oracle (oracle/attention.py)."""
import numpy as np
import pytest
import torch

from oracle import attention as oa


def _case(B, T, Hq, Hkv, Dh, ctx, bs, seed, shuffle=True):
    g = np.random.default_rng(seed)
    n_tok = [c + T for c in ctx]
    nblk = [-(-n // bs) for n in n_tok]
    num_blocks = sum(nblk) + 3
    ids = g.permutation(num_blocks) if shuffle else np.arange(num_blocks)
    table = np.zeros((B, max(nblk)), np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = ids[o:o + nblk[b]]
        o += nblk[b]
    kc = g.standard_normal((num_blocks, Hkv, bs, Dh))
    vc = g.standard_normal((num_blocks, Hkv, Dh, bs))
    q = g.standard_normal((B, T, Hq, Dh))
    return q, kc, vc, table, np.array(ctx, np.int32)


@pytest.mark.parametrize("B,T,Hq,Hkv,Dh,ctx", [(2, 5, 8, 2, 16, [7, 40]), (1, 1, 4, 4, 8, [0]),
                                                (3, 3, 6, 1, 32, [33, 1, 64])])
def test_matches_torch_sdpa_on_contiguous_cache(B, T, Hq, Hkv, Dh, ctx):
    bs = 8
    q, kc, vc, table, ctx = _case(B, T, Hq, Hkv, Dh, list(ctx), bs, 1, shuffle=False)
    scale = 1.0 / np.sqrt(Dh)
    out = oa.attention(q, kc, vc, table, ctx, bs, scale)
    G = Hq // Hkv
    for b in range(B):
        n = int(ctx[b]) + T
        k, v = oa.gather(kc, vc, table[b], n, bs)
        kk = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)      # [Hq, n, Dh]
        vv = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
        qq = torch.from_numpy(q[b]).permute(1, 0, 2)                           # [Hq, T, Dh]
        mask = torch.ones(T, n, dtype=torch.bool)
        for t in range(T):
            mask[t, int(ctx[b]) + t + 1:] = False
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
        assert np.allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_block_placement_does_not_matter():
    q, kc, vc, table, ctx = _case(2, 4, 4, 2, 16, [20, 3], 8, 5, shuffle=False)
    ref = oa.attention(q, kc, vc, table, ctx, 8, 0.25)
    g = np.random.default_rng(9)
    perm = g.permutation(kc.shape[0])                 # new physical id of every block
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    table2 = perm[table]
    assert np.array_equal(oa.attention(q, kc2, vc2, table2, ctx, 8, 0.25), ref)


def test_zero_query_averages_visible_values_and_single_key_returns_it():
    q, kc, vc, table, ctx = _case(1, 3, 2, 1, 8, [5], 4, 2)
    q[:] = 0.0
    out = oa.attention(q, kc, vc, table, ctx, 4, 1.0)
    k, v = oa.gather(kc, vc, table[0], 8, 4)
    for t in range(3):
        assert np.allclose(out[0, t, 0], v[:5 + t + 1, 0].mean(0))
    q2, kc2, vc2, table2, ctx2 = _case(1, 1, 3, 3, 8, [0], 4, 3)
    out2 = oa.attention(q2, kc2, vc2, table2, ctx2, 4, 1.0)
    _, v2 = oa.gather(kc2, vc2, table2[0], 1, 4)
    assert np.allclose(out2[0, 0], v2[0])


def test_append_commit_rollback_cycle():
    """A step appends T positions; after acceptance the committed prefix is
    ctx + AL, and the next step's attention depends only on it: whatever the
    rejected slots held is overwritten, and trimmed blocks come back."""
    g = np.random.default_rng(4)
    B, T, Hkv, Dh, bs = 2, 5, 2, 8, 4
    pool = oa.BlockPool(16)
    rows = [[], []]
    ctx = np.array([6, 1], np.int32)
    kc = np.zeros((16, Hkv, bs, Dh))
    vc = np.zeros((16, Hkv, Dh, bs))
    for b in range(B):                                   # prefill the committed prefix
        pool.reserve(rows[b], int(ctx[b]), bs, 8)
        for p in range(int(ctx[b])):
            kc[rows[b][p // bs], :, p % bs] = g.standard_normal((Hkv, Dh))
            vc[rows[b][p // bs], :, :, p % bs] = g.standard_normal((Hkv, Dh))
    assert pool.free[-1] == 3 and len(pool.free) == 16 - 3
    for b in range(B):
        pool.reserve(rows[b], int(ctx[b]) + T, bs, 8)
    table = np.array([r + [0] * (8 - len(r)) for r in rows], np.int32)
    kn, vn = g.standard_normal((B, T, Hkv, Dh)), g.standard_normal((B, T, Hkv, Dh))
    oa.append(kn, vn, kc, vc, table, ctx, bs)
    al = np.array([2, 5])
    new_ctx = oa.commit(ctx, al)
    assert new_ctx.tolist() == [8, 6]
    free_before = len(pool.free)
    for b in range(B):
        pool.trim(rows[b], int(new_ctx[b]), bs)
    assert [len(r) for r in rows] == [2, 2] and len(pool.free) == free_before + 1
    # the next step over the committed prefix: garbage in the freed slots is irrelevant
    q = g.standard_normal((B, 1, 2 * Hkv, Dh))
    table = np.array([r + [0] * (8 - len(r)) for r in rows], np.int32)
    for b in range(B):
        pool.reserve(rows[b], int(new_ctx[b]) + 1, bs, 8)
    table = np.array([r + [0] * (8 - len(r)) for r in rows], np.int32)
    kn1, vn1 = g.standard_normal((B, 1, Hkv, Dh)), g.standard_normal((B, 1, Hkv, Dh))
    kc_a, vc_a = kc.copy(), vc.copy()
    oa.append(kn1, vn1, kc_a, vc_a, table, new_ctx, bs)
    out_a = oa.attention(q, kc_a, vc_a, table, new_ctx, bs, 0.3)
    # scribble over every slot past each committed prefix, then append again
    kc_b, vc_b = kc.copy(), vc.copy()
    for b in range(B):
        for p in range(int(new_ctx[b]), len(rows[b]) * bs):
            kc_b[rows[b][p // bs], :, p % bs] = 1e3
            vc_b[rows[b][p // bs], :, :, p % bs] = -1e3
    oa.append(kn1, vn1, kc_b, vc_b, table, new_ctx, bs)
    assert np.array_equal(oa.attention(q, kc_b, vc_b, table, new_ctx, bs, 0.3), out_a)


def test_commit_skips_invalid_and_pool_limits():
    assert oa.commit([3, 4, 5], [0, 1, 3]).tolist() == [3, 5, 8]
    pool = oa.BlockPool(2)
    row = []
    with pytest.raises(MemoryError):
        pool.reserve(row, 9, 4, 8)
    pool.reserve(row, 8, 4, 8)
    assert row == [0, 1] and pool.free == []
    pool.trim(row, 0, 4)
    assert row == [] and pool.free == [1, 0]
