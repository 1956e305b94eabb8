"""GPU parity of the rejection-sampling stage (spec_verify_accept).

Both sides read the same fp32 logits and draft tokens (from ``workload`` and
the oracle's draft sampler), so tokens and acceptance lengths must match
bit for bit except requests with a decision inside the 1e-5 band.
"""
import numpy as np
import pytest
import torch
from scipy.stats import chisquare

import workload
from oracle import laws, verify as ov
from tests.gpu_helpers import compare_accept, cpu, gpu, note, require_gpu

CASES = [
    # B, K, V, T, scale, sigma  (ragged V, K = 0, long K, full-size vocab shapes)
    (1, 4, 4096, 1.0, 1.0, 0.5),
    (3, 2, 1001, 1.0, 1.3, 0.4),
    (5, 0, 777, 0.8, 1.3, 0.3),
    (2, 8, 513, 1.0, 2.0, 1.0),
    (16, 4, 32000, 1.0, 1.28, 0.38),       # 8B-shaped vocabulary, sigma 0.3
    (8, 4, 128256, 1.0, 1.81, 0.54),       # 70B-share shape
    (8, 4, 128256, 0.0, 1.81, 0.54),       # ... greedy
    (256, 2, 128256, 0.7, 1.28, 0.64),     # large batch, T = 0.7
    (7, 3, 2053, 0.0, 1.0, 0.5),
    (4, 3, 3000, 3.0, 1.0, 2.0),           # high temperature: acceptance collapse
    (3, 20, 5000, 1.0, 1.5, 0.2),          # long drafts: five positions per wave
    (1024, 1, 4096, 1.0, 1.5, 0.4),        # many short requests: 1024 chunk groups, split form
    (4, 4, 3000, 0.05, 1.5, 0.3),          # sharp: most probabilities underflow to zero
    (3, 3, 1, 1.0, 1.0, 0.5),              # one-token vocabulary: p = q = 1
    (3, 3, 1, 0.0, 1.0, 0.5),
    (5, 2, 2, 1.0, 1.0, 1.0),              # two tokens
    (5, 2, 3, 0.0, 1.0, 1.0),
]


def _run_case(sv, B, K, V, T, scale, sigma, seed, step):
    t, d = workload.make_synthetic_logits(B, K, V, scale, sigma, seed=seed)
    x = ov.sample_draft_tokens(d, T, seed, step)
    ref_out, ref_al, res = ov.verify(t, d, x, T, seed, step)
    tt, dd, xx = torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(), torch.from_numpy(x).cuda()
    p_at = torch.empty((B, K), dtype=torch.float32, device="cuda")
    q_at = torch.empty((B, K), dtype=torch.float32, device="cuda")
    out, al = sv.accept(tt, dd if K else None, xx if K else None, T, seed, step, p_at=p_at, q_at=q_at)
    torch.cuda.synchronize()
    return cpu(out), cpu(al), ref_out, ref_al, res, cpu(p_at), cpu(q_at), t, d, x


@gpu
@pytest.mark.parametrize("B,K,V,T,scale,sigma", CASES)
def test_accept_matches_oracle(B, K, V, T, scale, sigma):
    sv = require_gpu()
    note(f"accept parity B={B} K={K} V={V} T={T}")
    for seed, step in ((0, 0), (7, 3)):
        go, ga, ro, ra, res, p_at, q_at, t, d, x = _run_case(sv, B, K, V, T, scale, sigma, seed, step)
        near = compare_accept(go, ga, ro, ra, res)
        assert np.all((ga >= 1) & (ga <= K + 1))
        if T > 0 and K > 0:
            # p(x), q(x) against the oracle's fp64 softmax: fp32 sums and the exp unit
            # (relative error ~ 2^-24 * |exponent * log2 e| + 1 ulp) stay within 5e-6
            for b in range(min(B, 8)):
                for j in range(K):
                    p = ov.softmax(t[b, j], T)[x[b, j]]
                    q = ov.softmax(d[b, j], T)[x[b, j]]
                    assert abs(p_at[b, j] - p) <= 5e-6 * p + 1e-30
                    assert abs(q_at[b, j] - q) <= 5e-6 * q + 1e-30
        note(f"  seed={seed} step={step}: {B - near}/{B} requests compared, {near} near-threshold")


@gpu
def test_p_equals_q_full_acceptance():
    sv = require_gpu()
    B, K, V = 64, 4, 5000
    t, _ = workload.make_synthetic_logits(B, K, V, 1.5, 0.0, seed=3)
    d = np.ascontiguousarray(t[:, :K])
    for step in range(3):
        x = ov.sample_draft_tokens(d, 1.0, 3, step)
        out, al = sv.accept(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(),
                            torch.from_numpy(x).cuda(), 1.0, 3, step)
        al = cpu(al)
        assert np.all(al == K + 1)
        assert np.array_equal(cpu(out)[:, :K], x)


@gpu
def test_disjoint_supports_reject_first():
    sv = require_gpu()
    B, K, V = 32, 3, 4000
    t = np.zeros((B, K + 1, V), np.float32)
    d = np.zeros((B, K, V), np.float32)
    t[:, :, : V // 2] = -1e4
    d[:, :, V // 2:] = -1e4
    x = ov.sample_draft_tokens(d, 1.0, 1, 0)
    out, al = sv.accept(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(),
                        torch.from_numpy(x).cuda(), 1.0, 1, 0)
    assert np.all(cpu(al) == 1)
    assert np.all(cpu(out)[:, 0] >= V // 2)


@gpu
def test_invalid_draft_tokens_give_sentinel():
    sv = require_gpu()
    B, K, V = 4, 3, 100
    t, d = workload.make_synthetic_logits(B, K, V, 1.0, 0.5, seed=2)
    x = ov.sample_draft_tokens(d, 1.0, 2, 0)
    x[0, 1] = V
    x[2, 0] = -5
    for T in (1.0, 0.0):
        out, al = sv.accept(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(),
                            torch.from_numpy(x).cuda(), T, 2, 0)
        out, al = cpu(out), cpu(al)
        assert al[0] == 0 and al[2] == 0 and np.all(out[[0, 2]] == -1)
        assert al[1] >= 1 and al[3] >= 1


@gpu
def test_greedy_is_argmax_prefix():
    sv = require_gpu()
    B, K, V = 100, 4, 3001
    t, d = workload.make_synthetic_logits(B, K, V, 1.0, 0.5, seed=9)
    greedy = t.argmax(-1)
    x = greedy[:, :K].astype(np.int32).copy()
    g = np.random.default_rng(1)
    flip = g.random((B, K)) < 0.25
    x[flip] = (x[flip] + 1) % V
    out, al = sv.accept(torch.from_numpy(t).cuda(), None, torch.from_numpy(x).cuda(), 0.0, 0, 0)
    out, al = cpu(out), cpu(al)
    for b in range(B):
        m = 0
        while m < K and x[b, m] == greedy[b, m]:
            m += 1
        assert al[b] == m + 1 and np.array_equal(out[b, :al[b]], greedy[b, :al[b]])


@gpu
def test_deterministic_reruns():
    sv = require_gpu()
    B, K, V = 64, 4, 32000
    t, d = workload.make_synthetic_logits(B, K, V, 1.3, 0.4, seed=4)
    x = ov.sample_draft_tokens(d, 1.0, 4, 0)
    args = (torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(), torch.from_numpy(x).cuda())
    o1, a1 = sv.accept(*args, 1.0, 4, 0)
    o2, a2 = sv.accept(*args, 1.0, 4, 0)
    assert torch.equal(o1, o2) and torch.equal(a1, a2)
    o3, _ = sv.accept(*args, 1.0, 4, 1)     # a new step draws new uniforms
    assert not torch.equal(o1, o3)


@gpu
@pytest.mark.parametrize("V,K,T", [(4, 2, 1.0), (3, 3, 0.8), (6, 1, 1.0), (5, 0, 1.0)])
def test_kernel_law_chi2(V, K, T):
    """Emitted tuples over 2^17 requests vs the exact law (enumeration)."""
    sv = require_gpu()
    n = 1 << 17
    g = np.random.default_rng(V * 10 + K)
    zt = g.standard_normal((K + 1, V)).astype(np.float32)
    zd = (zt[:K] + 0.8 * g.standard_normal((K, V))).astype(np.float32)
    p, q = ov.softmax(zt.astype(np.float64), T), ov.softmax(zd.astype(np.float64), T)
    law = laws.exact_outcome_law(p, q)
    x = np.stack([g.choice(V, size=n, p=q[j]) for j in range(K)], 1).astype(np.int32) if K else \
        np.zeros((n, 0), np.int32)
    tt = torch.from_numpy(np.broadcast_to(zt, (n, K + 1, V)).copy()).cuda()
    dd = torch.from_numpy(np.broadcast_to(zd, (n, K, V)).copy()).cuda()
    out, al = sv.accept(tt, dd if K else None, torch.from_numpy(x).cuda() if K else None, T, 11, 5)
    out, al = cpu(out), cpu(al)
    keys = {}
    for b in range(n):
        k = tuple(out[b, :al[b]].tolist())
        keys[k] = keys.get(k, 0) + 1
    assert set(keys) <= set(law)
    ks = sorted(law, key=lambda k: -law[k])
    e = np.array([law[k] * n for k in ks])
    o = np.array([keys.get(k, 0) for k in ks], float)
    big = e >= 5
    e2, o2 = np.append(e[big], e[~big].sum()), np.append(o[big], o[~big].sum())
    if e2[-1] < 5:
        e2, o2 = e2[:-1], o2[:-1]
    pv = chisquare(o2, e2 * o2.sum() / e2.sum()).pvalue
    note(f"chi2 V={V} K={K}: p = {pv:.3g}")
    assert pv > 1e-4


@gpu
@pytest.mark.parametrize("B,K,V,T", [(1, 4, 4096, 1.0), (24, 3, 9001, 0.7), (64, 4, 32000, 1.0),
                                     (256, 2, 128256, 0.7), (8, 4, 128256, 0.0), (5, 0, 777, 0.8),
                                     (3, 2, 1001, 3.0), (8, 4, 128256, 1.0), (2, 16, 70000, 1.0)])
def test_split_and_fused_decisions_agree(B, K, V, T, monkeypatch):
    """The stage's two launch forms -- decisions taken in every chunk
    workgroup (one launch), or once per request and then the chunk totals
    (two launches) -- run the same arithmetic on the same values, so they
    agree bit for bit: tokens, acceptance lengths, p(x) and q(x)."""
    sv = require_gpu()
    t, d = workload.make_synthetic_logits(B, K, V, 1.3, 0.4, seed=11)
    x = ov.sample_draft_tokens(d, T, 11, 2)
    tt, dd, xx = torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(), torch.from_numpy(x).cuda()
    got = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("SPEC_VERIFY_ACCEPT_SPLIT", mode)
        p_at = torch.full((B, K), float("nan"), dtype=torch.float32, device="cuda")
        q_at = torch.full((B, K), float("nan"), dtype=torch.float32, device="cuda")
        out, al = sv.accept(tt, dd if K else None, xx if K else None, T, 11, 2, p_at=p_at, q_at=q_at)
        torch.cuda.synchronize()
        got[mode] = (cpu(out), cpu(al), cpu(p_at).view(np.int32), cpu(q_at).view(np.int32))
    for a, b in zip(got["0"], got["1"]):
        assert np.array_equal(a, b)
    note(f"split vs fused B={B} K={K} V={V} T={T}: identical; AL {got['1'][1][:8].tolist()}")
