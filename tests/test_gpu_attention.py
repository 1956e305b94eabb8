"""GPU parity of the paged attention of the verified positions
(include/spec_verify_attn.h) against oracle/attention.py.

Inputs from ``workload.make_paged_attention`` (seeded, physically shuffled
blocks).  Tolerance: both sides read the same bf16 values and the scores are
fp32 sums of exact products, so the difference comes from the
probabilities entering the value product rounded to bf16 (relative error
<= 2^-9 each) with the softmax sum taken over the same rounded values: the
output is then a convex combination whose weights are each off by at most
2 * 2^-9 relative, i.e. |out - ref| <= 2^-8 * max |v| (+ fp32 rounding).
Cache writes (append) and the commit are bit-exact.
"""
import numpy as np
import pytest
import torch

import workload
from oracle import attention as oa
from tests.gpu_helpers import cpu, gpu, note, require_gpu

TOL_REL_V = 2.0 ** -8


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bits(t):
    """bf16 device tensor -> its uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _f32(a):
    return workload.bf16_bits_to_f32(a).astype(np.float64)


def _run(sv, case, T, scale):
    kc, vc = _dev(case["k_cache"]), _dev(case["v_cache"])
    table, ctx = _dev(case["block_table"]), _dev(case["ctx_len"])
    sv.kv_append(_dev(case["k_new"]), _dev(case["v_new"]), kc, vc, table, ctx)
    out = sv.attention(_dev(case["q"]), kc, vc, table, ctx, scale)
    torch.cuda.synchronize()
    return cpu(out), kc, vc


def _reference(case, T, scale):
    kc, vc = _f32(case["k_cache"]), _f32(case["v_cache"])
    oa.append(_f32(case["k_new"]), _f32(case["v_new"]), kc, vc, case["block_table"],
              case["ctx_len"], workload.KV_BLOCK)
    return oa.attention(_f32(case["q"]), kc, vc, case["block_table"], case["ctx_len"],
                        workload.KV_BLOCK, scale), kc, vc


CASES = [
    # B, T, Hq, Hkv, Dh, ctx per request, max_blocks
    (1, 1, 8, 8, 128, [0], 1),                   # a single key: the step's own position
    (2, 5, 32, 8, 128, [7, 100], 4),             # 8B-shaped heads, ragged, partial blocks
    (3, 3, 8, 1, 64, [31, 32, 33], 2),           # multi-query, block boundaries
    (2, 9, 16, 2, 128, [500, 3], 16),            # G*T = 72 rows: several query tiles
    (4, 5, 64, 8, 128, [1000, 2000, 1, 64], 64), # 70B-shaped heads, split context
    (1, 2, 4, 4, 64, [4000], 126),               # long context, G = 1
    (5, 1, 12, 4, 128, [10, 20, 30, 40, 50], 2), # T = 1 (no drafts)
    (2, 16, 8, 1, 64, [300, 50], 12),            # 128 rows per KV head: 8 tiles (ring)
    (1, 16, 64, 8, 128, [700], 24),              # 70B-shaped heads, K = 15: 8 tiles, split
    (2, 8, 8, 1, 128, [64, 500], 18),            # 4 tiles: the LDS-ring kernel, one tile per wave
    (1, 16, 16, 1, 64, [200], 8),                # 16 tiles: ring, four tiles per wave
    (2, 16, 8, 1, 64, [1500, 40], 64),           # head_dim 64, two tiles per wave, 8 context splits
    (1, 16, 16, 1, 64, [2000], 72),              # head_dim 64, four tiles per wave, 9 context splits
]


@gpu
@pytest.mark.parametrize("B,T,Hq,Hkv,Dh,ctx,mb", CASES)
def test_attention_matches_oracle(B, T, Hq, Hkv, Dh, ctx, mb):
    sv = require_gpu()
    note(f"attention B={B} T={T} Hq={Hq} Hkv={Hkv} Dh={Dh} ctx={ctx} max_blocks={mb}")
    case = workload.make_paged_attention(B, T, Hq, Hkv, Dh, ctx, mb, seed=B * 100 + T)
    scale = 1.0 / np.sqrt(Dh)
    got, kc, vc = _run(sv, case, T, scale)
    ref, rk, rv = _reference(case, T, scale)
    # the appended cache is bit-exact
    assert np.array_equal(workload.bf16_bits_to_f32(_bits(kc)), rk.astype(np.float32))
    assert np.array_equal(workload.bf16_bits_to_f32(_bits(vc)), rv.astype(np.float32))
    vmax = float(np.abs(rv).max())
    err = np.abs(got - ref).max()
    note(f"  max |out - ref| = {err:.3g} (tol {TOL_REL_V * vmax:.3g})")
    assert np.all(np.isfinite(got))
    assert err <= TOL_REL_V * vmax + 1e-6


@gpu
def test_commit_and_rollback_cycle():
    """Append, attend, commit AL on the device, trim the host tables through
    the library's block pool, then attend again: equal to the oracle's cycle,
    and the rejected slots' contents do not matter."""
    sv = require_gpu()
    B, T, Hq, Hkv, Dh = 3, 5, 16, 4, 128
    ctx0 = np.array([40, 0, 95], np.int32)
    mb = 8
    pool = sv.KVPool(64)
    ref_pool = oa.BlockPool(64)
    rows = np.zeros((B, mb), np.int32)
    nblk = [0] * B
    ref_rows = [[] for _ in range(B)]
    for b in range(B):
        nblk[b] = pool.reserve(rows[b], nblk[b], int(ctx0[b]) + T)
        ref_pool.reserve(ref_rows[b], int(ctx0[b]) + T, workload.KV_BLOCK, mb)
        assert rows[b, :nblk[b]].tolist() == ref_rows[b]
    g = np.random.default_rng(3)
    nb = 64
    kc = workload.f32_to_bf16_bits(g.standard_normal((nb, Hkv, 32, Dh)).astype(np.float32))
    vc = workload.f32_to_bf16_bits(g.standard_normal((nb, Hkv, Dh, 32)).astype(np.float32))
    mk = lambda *s: workload.f32_to_bf16_bits(g.standard_normal(s).astype(np.float32))
    q1, kn1, vn1 = mk(B, T, Hq, Dh), mk(B, T, Hkv, Dh), mk(B, T, Hkv, Dh)
    dkc, dvc, dtab, dctx = _dev(kc), _dev(vc), _dev(rows), _dev(ctx0)
    sv.kv_append(_dev(kn1), _dev(vn1), dkc, dvc, dtab, dctx)
    sv.attention(_dev(q1), dkc, dvc, dtab, dctx, 0.1)
    al = np.array([2, 5, 0], np.int32)                   # the last request was invalid
    sv.kv_commit(dctx, _dev(al))
    new_ctx = cpu(dctx)
    assert new_ctx.tolist() == oa.commit(ctx0, al).tolist() == [42, 5, 95]
    free0 = pool.free_blocks
    for b in range(B):
        nblk[b] = pool.trim(rows[b], nblk[b], int(new_ctx[b]))
        ref_pool.trim(ref_rows[b], int(new_ctx[b]), workload.KV_BLOCK)
        assert rows[b, :nblk[b]].tolist() == ref_rows[b]
    assert pool.free_blocks == len(ref_pool.free) and pool.free_blocks >= free0
    # next step: one new position per request
    for b in range(B):
        nblk[b] = pool.reserve(rows[b], nblk[b], int(new_ctx[b]) + 1)
        ref_pool.reserve(ref_rows[b], int(new_ctx[b]) + 1, workload.KV_BLOCK, mb)
        assert rows[b, :nblk[b]].tolist() == ref_rows[b]
    q2, kn2, vn2 = mk(B, 1, Hq, Dh), mk(B, 1, Hkv, Dh), mk(B, 1, Hkv, Dh)
    dtab = _dev(rows)
    sv.kv_append(_dev(kn2), _dev(vn2), dkc, dvc, dtab, dctx)
    out = cpu(sv.attention(_dev(q2), dkc, dvc, dtab, dctx, 0.1))
    rk, rv = _f32(kc), _f32(vc)
    oa.append(_f32(kn1), _f32(vn1), rk, rv, rows, ctx0, 32)
    oa.append(_f32(kn2), _f32(vn2), rk, rv, rows, new_ctx, 32)
    ref = oa.attention(_f32(q2), rk, rv, rows, new_ctx, 32, 0.1)
    assert np.abs(out - ref).max() <= TOL_REL_V * np.abs(rv).max() + 1e-6


@gpu
def test_out_of_range_block_ids_are_clamped():
    """Table entries outside [0, num_blocks) read a clamped block instead of
    memory outside the cache (the host never reads device tables).  The bad
    entries sit at read-only block indices, so no two appends meet."""
    sv = require_gpu()
    case = workload.make_paged_attention(2, 3, 8, 2, 64, [40, 40], 4, seed=11)
    nb = case["num_blocks"]
    bad = case["block_table"].copy()
    bad[0, 0] = -7
    bad[1, 0] = nb + 100
    got, _, _ = _run(sv, dict(case, block_table=bad), 3, 0.125)
    ref, _, rv = _reference(dict(case, block_table=np.clip(bad, 0, nb - 1)), 3, 0.125)
    assert np.abs(got - ref).max() <= TOL_REL_V * np.abs(rv).max() + 1e-6
