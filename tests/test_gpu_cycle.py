"""GPU parity of the speculative cycle (include/spec_verify_cycle.h) against
oracle/cycle.py: the embedding gather, the draft-token sampler, the draft
loop, whole cycles, plain decoding (K = 0) and a graph-captured cycle.

Tokens are compared bit for bit.  A request is set aside (and counted) only
where a logit error of the measured size could move one of its decisions: a
draft draw whose threshold lies within (2 eps / T + 1e-5) of a CDF boundary
(relative to the total), or a verification decision inside the band of
tests/gpu_helpers.step_band_near.  eps is measured: the GPU forward of the
same rows (the oracle's tokens) against the oracle's logits, with a factor of
4 for the other row counts inside the cycle.  The target and drafter are
fp32 stacks, whose logits match the oracle within 1e-4.
"""
import numpy as np
import pytest
import torch

import workload
from oracle import cycle as oc
from oracle import forward as of
from tests.gpu_helpers import TOL_F32, cpu, device_model, gpu, note, require_gpu, step_band_near

EPS = TOL_F32


def _models(sv, sigma=0.6, L=2, V=1001, ffn=1024):
    w = workload.Workload("cycle-f32", 256, ffn, L, V, "f32", 1, 4, sigma, 1.0, "var_inv_d", 21)
    model = workload.make_model(w)
    drafter = of.truncated(model, 1)
    drafter["w_head"] = model["w_draft_head"]
    table = workload.make_embedding(w)
    return (w, model, drafter, table, device_model(sv, model), device_model(sv, drafter),
            torch.from_numpy(table).cuda())


def _draw_near(d: oc.DraftDraw, T: float, eps: float) -> bool:
    """Whether a logit error of at most eps can move the draft draw d."""
    if T == 0.0:
        return d.margin <= 2 * eps + 1e-6
    return d.margin <= 2 * eps / T + 1e-5


def _measured_eps(d_model, d_drafter, d_table, start, r: oc.CycleResult):
    """Per request: 4 x the largest |GPU - oracle| logit over its target rows
    (eps_t) and over its draft rows (eps_d), the GPU forwards run on the
    oracle's tokens."""
    B, K1, V = r.target_logits.shape
    K = K1 - 1
    toks = np.concatenate([np.asarray(start, np.int32)[:, None], r.draft_tokens], axis=1)
    zt = cpu(d_model.forward(d_table[torch.from_numpy(toks.reshape(-1)).long().cuda()].contiguous()))
    eps_t = 4 * np.abs(zt.reshape(B, K1, V) - r.target_logits).max(axis=(1, 2))
    eps_d = np.zeros(B)
    if K:
        zd = cpu(d_drafter.forward(d_table[torch.from_numpy(toks[:, :K].reshape(-1)).long().cuda()]
                                   .contiguous()))
        eps_d = 4 * np.abs(zd.reshape(B, K, V) - r.draft_logits).max(axis=(1, 2))
    return eps_t, eps_d


@gpu
def test_embed_gathers_rows_and_zeroes_bad_tokens():
    sv = require_gpu()
    w = workload.Workload("emb", 64, 128, 1, 1001, "f32", 1, 1, 0.1, 1.0, "var_inv_d", 2)
    table = workload.make_embedding(w)
    tok = np.array([0, 1000, 17, -1, 1001, 5000, 17], dtype=np.int32)
    out = cpu(sv.embed(torch.from_numpy(table).cuda(), torch.from_numpy(tok).cuda()))
    assert np.array_equal(out, oc.embed(table, tok).astype(np.float32))


@gpu
@pytest.mark.parametrize("V", [1001, 20000])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_sample_matches_the_oracle_draws(V, T):
    """One draft-slot draw per row (several 8192-logit chunks at V = 20000),
    written with a stride into a wider array.  The logits spread like a
    language model's (a few dozen likely tokens), so most draws sit well away
    from the stated 1e-5 band."""
    sv = require_gpu()
    B, stride, slot = 96, 3, 4
    z = workload.make_synthetic_logits(B, 0, V, 2.5, 0.0, seed=V, sub=int(T * 10))[0][:, 0]
    out = torch.full((B * stride,), -7, dtype=torch.int32, device="cuda")
    sv.sample(torch.from_numpy(np.ascontiguousarray(z)).cuda(), T, 77, 5, slot, tokens=out[1:],
              out_stride=stride)
    got = cpu(out).reshape(B, stride)
    assert (got[:, 0] == -7).all() and (got[:, 2] == -7).all()
    near = 0
    for b in range(B):
        # identical logits on both sides: only the fp32 softmax differs
        d = oc.draw_token(z[b], T, b, slot, 77, 5)
        if _draw_near(d, T, 0.0):
            near += 1
            continue
        assert got[b, 1] == d.token, (b, got[b, 1], d.token)
    note(f"  sample V={V} T={T}: {B - near} rows bit-exact, {near} near a boundary")
    assert near <= B // 2


@gpu
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_draft_loop_matches_the_oracle(T):
    sv = require_gpu()
    w, model, drafter, table, _, d_drafter, d_table = _models(sv)
    B, K = 6, 5
    cur = workload.make_start_tokens(w.vocab, B, seed=3)
    x, zq = d_drafter.draft(d_table, torch.from_numpy(cur).cuda(), K, T, 9, 2)
    x, zq = cpu(x), cpu(zq)
    ref_x, ref_zq, draws = oc.draft(drafter, table, cur, K, T, 9, 2)
    compared = 0
    for b in range(B):
        for j in range(K):
            # the slot's input is the same on both sides while the tokens agree
            err = np.abs(zq[b, j] - ref_zq[b, j]).max()
            assert err <= EPS
            if _draw_near(draws[b][j], T, 4 * err):
                break
            assert x[b, j] == ref_x[b, j], (b, j)
            compared += 1
    note(f"  draft loop T={T}: {compared} of {B * K} draws compared bit-exactly")
    assert compared >= B * K * 3 // 4


@gpu
@pytest.mark.parametrize("K,T", [(4, 1.0), (3, 0.7), (4, 0.0), (0, 1.0)])
def test_cycles_match_the_oracle(K, T):
    """Three cycles in a row; each is compared with the oracle started from
    the GPU's current tokens, so one set-aside request does not hide the
    next cycle."""
    sv = require_gpu()
    w, model, drafter, table, d_model, d_drafter, d_table = _models(sv)
    B = 8
    cur = torch.from_numpy(workload.make_start_tokens(w.vocab, B, seed=5)).cuda()
    aside = total = 0
    for step in range(3):
        start = cpu(cur).copy()
        out, al = sv.cycle(d_model, d_drafter if K else None, d_table, cur, K, T, 31, step)
        out, al, nxt = cpu(out), cpu(al), cpu(cur)
        r = oc.cycle(model, drafter, table, start, K, T, 31, step)
        eps_t, eps_d = _measured_eps(d_model, d_drafter, d_table, start, r)
        assert eps_t.max() <= 4 * EPS and eps_d.max() <= 4 * EPS
        for b in range(B):
            total += 1
            if any(_draw_near(d, T, eps_d[b]) for d in r.draft_draws[b]) or \
                    step_band_near(r.results[b], eps_t[b] + eps_d[b], T, r.target_logits[b]):
                aside += 1
                continue
            assert al[b] == r.accept_len[b], (step, b, al[b], r.accept_len[b])
            assert np.array_equal(out[b], r.out_tokens[b]), (step, b)
            assert nxt[b] == r.next_cur[b]
        if K == 0:
            assert (al == 1).all()
    note(f"  cycles K={K} T={T}: {total - aside} request-cycles bit-exact, {aside} set aside")
    assert aside <= total // 4


@gpu
def test_drafter_equal_to_target_accepts_every_draft():
    """A bf16 target drafting for itself: the draft rows (2 positions per
    pass) and the verified rows (8) run the same kernels, so p = q bit for bit
    and every draft is accepted."""
    sv = require_gpu()
    w = workload.Workload("cycle-bf16", 256, 768, 2, 1001, "bf16", 1, 3, 0.3, 1.0, "std_0.02", 4)
    model = workload.make_model(w, draft_head=False)
    d_model = device_model(sv, model, tiled=True)
    table = torch.from_numpy(workload.make_embedding(w)).cuda()
    cur = torch.from_numpy(workload.make_start_tokens(w.vocab, 2, seed=8)).cuda()
    for step in range(4):
        out, al = sv.cycle(d_model, d_model, table, cur, 3, 1.0, 3, step)
        assert (cpu(al) == 4).all()
        assert (cpu(out) >= 0).all() and (cpu(out) < w.vocab).all()


@gpu
def test_graph_replays_of_a_cycle_equal_eager():
    """The whole cycle captured once; every replay (current tokens reset by
    eager work between replays) matches the eager cycle."""
    sv = require_gpu()
    w, model, drafter, table, d_model, d_drafter, d_table = _models(sv)
    B, K, T = 4, 3, 1.0
    start = torch.from_numpy(workload.make_start_tokens(w.vocab, B, seed=9)).cuda()
    cur = start.clone()
    ws = sv.workspace(sv.cycle_workspace_bytes(d_model, d_drafter, B, K))
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    sv.cycle(d_model, d_drafter, d_table, cur, K, T, 5, 1, out, al, ws)
    torch.cuda.synchronize()
    ref = (cpu(out).copy(), cpu(al).copy(), cpu(cur).copy())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    cur.copy_(start)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        sv.cycle(d_model, d_drafter, d_table, cur, K, T, 5, 1, out, al, ws, stream=s)
    for _ in range(3):
        cur.copy_(start)
        out.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(cpu(out), ref[0]) and np.array_equal(cpu(al), ref[1])
        assert np.array_equal(cpu(cur), ref[2])
