"""Pins for the oracle's modified rejection sampling.

Each test checks the oracle against something the pages or the mathematics
fix, not against a retyping of the oracle's own code.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import binomtest, chisquare

import workload
from oracle import laws, philox, verify as ov

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _dists(V, K, seed, spread=1.0, sigma=0.7):
    g = np.random.default_rng(seed)
    zt = g.standard_normal((K + 1, V)) * spread
    zd = zt[:K] + sigma * g.standard_normal((K, V))
    return zt, zd


def _trials(zt, zd, T, n, seed=0):
    """n independent requests with the same distributions (request id b
    selects fresh counters); draft tokens drawn from q by the oracle."""
    K1, V = zt.shape
    K = K1 - 1
    tt = np.broadcast_to(zt, (n, K1, V))
    dd = np.broadcast_to(zd, (n, K, V))
    x = ov.sample_draft_tokens(dd, T, seed, 0)
    return ov.verify(tt, dd, x, T, seed, 0)


def _chi2(observed: dict, law: dict, n: int):
    keys = sorted(law, key=lambda k: -law[k])
    exp = np.array([law[k] * n for k in keys])
    obs = np.array([observed.get(k, 0) for k in keys], dtype=float)
    assert sum(observed.values()) == n and set(observed) <= set(law)
    # merge the tail so every bin expects at least 5
    big = exp >= 5
    e = np.append(exp[big], exp[~big].sum())
    o = np.append(obs[big], obs[~big].sum())
    if e[-1] < 5:
        e[-2] += e[-1]; o[-2] += o[-1]; e, o = e[:-1], o[:-1]
    return chisquare(o, e * o.sum() / e.sum()).pvalue


def test_al_range_and_padding():
    t, d = workload.make_synthetic_logits(64, 5, 300, 1.3, 0.6, seed=2)
    for T in (1.0, 0.7, 0.0):
        x = ov.sample_draft_tokens(d, T, 9, 0)
        out, al, _ = ov.verify(t, d, x, T, 9, 0)
        assert np.all((al >= 1) & (al <= 6))
        for b in range(64):
            assert np.all((out[b, :al[b]] >= 0) & (out[b, :al[b]] < 300))
            assert np.all(out[b, al[b]:] == -1)
            assert np.array_equal(out[b, :al[b] - 1], x[b, :al[b] - 1])   # accepted prefix


def test_p_equals_q_accepts_everything():
    g = np.random.default_rng(4)
    zt = g.standard_normal((40, 5, 50))
    zd = zt[:, :4].copy()
    for step in range(5):
        x = ov.sample_draft_tokens(zd, 1.0, 1, step)
        _, al, _ = ov.verify(zt, zd, x, 1.0, 1, step)
        assert np.all(al == 5)


def test_disjoint_supports_reject_first_draft():
    V, K, B = 40, 3, 30
    zt = np.zeros((B, K + 1, V)); zd = np.zeros((B, K, V))
    zt[:, :, : V // 2] = -1e4          # p lives on the upper half
    zd[:, :, V // 2:] = -1e4           # q lives on the lower half
    x = ov.sample_draft_tokens(zd, 1.0, 3, 0)
    assert np.all(x < V // 2)
    out, al, _ = ov.verify(zt, zd, x, 1.0, 3, 0)
    assert np.all(al == 1)
    assert np.all(out[:, 0] >= V // 2)  # replacement comes from max(0, p - q) = p


def test_greedy_reproduces_greedy_decoding():
    g = np.random.default_rng(5)
    B, K, V = 200, 4, 30
    zt = g.standard_normal((B, K + 1, V))
    greedy = zt.argmax(-1)                       # what plain greedy decoding emits
    x = greedy[:, :K].copy()
    flip = g.random((B, K)) < 0.3                # corrupt some drafts
    x[flip] = (x[flip] + 1 + g.integers(0, V - 1, flip.sum())) % V
    out, al, _ = ov.verify(zt, np.zeros((B, K, V)), x, 0.0, 0, 0)
    for b in range(B):
        match = 0
        while match < K and x[b, match] == greedy[b, match]:
            match += 1
        assert al[b] == match + 1
        assert np.array_equal(out[b, :al[b]], greedy[b, :al[b]])


def test_small_temperature_limit_is_greedy():
    g = np.random.default_rng(6)
    B, K, V = 50, 3, 20
    zt = g.standard_normal((B, K + 1, V))
    zd = zt[:, :K] + 0.5 * g.standard_normal((B, K, V))
    x = zd.argmax(-1).astype(np.int32)
    o0, a0, _ = ov.verify(zt, zd, x, 0.0, 0, 0)
    o1, a1, _ = ov.verify(zt, zd, x, 1e-4, 0, 0)
    assert np.array_equal(o0, o1) and np.array_equal(a0, a1)


def test_out_of_range_draft_is_flagged():
    zt, zd = _dists(10, 3, 0)
    x = np.array([[1, 10, 2], [-1, 0, 0], [1, 2, 3]])
    out, al, _ = ov.verify(np.stack([zt] * 3), np.stack([zd] * 3), x, 1.0, 0, 0)
    assert list(al[:2]) == [0, 0] and np.all(out[:2] == -1) and al[2] >= 1


@pytest.mark.parametrize("V,K,T", [(4, 2, 1.0), (3, 3, 0.8), (5, 1, 1.3)])
def test_exact_outcome_law_chi2(V, K, T):
    zt, zd = _dists(V, K, seed=V * 10 + K)
    law = laws.exact_outcome_law(ov.softmax(zt, T), ov.softmax(zd, T))
    assert abs(sum(law.values()) - 1.0) < 1e-12
    n = 12000
    out, al, _ = _trials(zt, zd, T, n, seed=K)
    obs = {}
    for b in range(n):
        key = tuple(int(v) for v in out[b, :al[b]])
        obs[key] = obs.get(key, 0) + 1
    assert _chi2(obs, law, n) > 1e-4


def test_emitted_marginal_is_target_distribution():
    # publishertech section 2: P(emit x) = min(p, q) + (p - min(p, q)) = p
    V, K, T = 6, 1, 1.0
    zt, zd = _dists(V, K, seed=11, sigma=1.5)
    p = ov.softmax(zt[0], T)
    law = laws.exact_outcome_law(ov.softmax(zt, T), ov.softmax(zd, T))
    marg = np.zeros(V)
    for k, v in law.items():
        marg[k[0]] += v
    assert np.allclose(marg, p, atol=1e-12)
    n = 20000
    out, _, _ = _trials(zt, zd, T, n, seed=5)
    counts = np.bincount(out[:, 0], minlength=V)
    assert chisquare(counts, p * n).pvalue > 1e-4


def test_acceptance_frequency_is_beta():
    V, K, T = 8, 1, 1.0
    zt, zd = _dists(V, K, seed=12, sigma=1.0)
    beta = laws.acceptance_prob(ov.softmax(zt[0], T), ov.softmax(zd[0], T))
    n = 20000
    _, al, _ = _trials(zt, zd, T, n, seed=6)
    assert binomtest(int((al == 2).sum()), n, beta).pvalue > 1e-4


def test_mean_al_matches_closed_form():
    # identical (p, q) at every position -> constant alpha = beta
    V, K, T = 12, 4, 1.0
    zt1, zd1 = _dists(V, 1, seed=13, sigma=0.6)
    zt = np.concatenate([np.repeat(zt1[:1], K, 0), zt1[1:]])
    zd = np.repeat(zd1, K, 0)
    beta = laws.acceptance_prob(ov.softmax(zt1[0], T), ov.softmax(zd1[0], T))
    n = 6000
    _, al, _ = _trials(zt, zd, T, n, seed=7)
    mean, se = al.mean(), al.std() / math.sqrt(n)
    assert abs(mean - laws.expected_tokens(beta, K)) < 4 * se
    assert abs(laws.expected_al([beta] * K) - laws.expected_tokens(beta, K)) < 1e-12
    assert chisquare(np.bincount(al, minlength=K + 2)[1:], laws.al_law([beta] * K) * n).pvalue > 1e-4


def test_k_zero_is_plain_sampling():
    V, T = 7, 0.9
    zt, _ = _dists(V, 0, seed=14)
    n = 20000
    out, al, _ = _trials(zt, np.zeros((0, V)), T, n, seed=8)
    assert np.all(al == 1)
    assert chisquare(np.bincount(out[:, 0], minlength=V), ov.softmax(zt[0], T) * n).pvalue > 1e-4


def test_residual_mass_identity():
    g = np.random.default_rng(15)
    for _ in range(20):
        p = ov.softmax(g.standard_normal(1000), 1.0)
        q = ov.softmax(g.standard_normal(1000), 1.0)
        assert abs(np.maximum(0, p - q).sum() - (1 - laws.acceptance_prob(p, q))) < 1e-12


def test_printed_speedup_values():
    with open(os.path.join(GOLDEN, "speedup_examples.json")) as f:
        gold = json.load(f)
    for e in gold["expected_tokens"]:
        assert round(laws.expected_tokens(e["alpha"], e["gamma"]), 2) in (e["printed"], e["printed"] + 0.01)
    for e in gold["expected_tokens_bracket"]:
        lo = laws.expected_tokens(e["alpha_lo"], e["gamma"])
        hi = laws.expected_tokens(e["alpha_hi"], e["gamma"])
        assert lo <= e["printed"] <= hi
    for e in gold["speedup"]:
        s = laws.speedup(e["expected_n"], e["gamma"], e["c"])
        if e["rounding"].startswith("exact"):
            assert round(s, 2) == e["printed"]
        else:
            assert math.floor(s * 100) / 100 == e["printed"]
    for e in gold["cycle_cost"]:
        assert 1 + e["gamma"] * e["c"] == e["printed_t_target_multiple"]


# --- planted mistakes: the pins above must catch them -----------------------

def test_planted_mistake_biased_accept_uniform_is_caught(monkeypatch):
    V, K, T = 8, 1, 1.0
    zt, zd = _dists(V, K, seed=12, sigma=1.0)
    beta = laws.acceptance_prob(ov.softmax(zt[0], T), ov.softmax(zd[0], T))
    monkeypatch.setattr(philox, "u_accept", lambda w: np.sqrt(
        ((np.asarray(w, np.uint64) >> np.uint64(8)) + np.uint64(1)).astype(np.float64) * 2.0 ** -24))
    _, al, _ = _trials(zt, zd, T, 20000, seed=6)
    assert binomtest(int((al == 2).sum()), 20000, beta).pvalue < 1e-6


def test_planted_mistake_reversed_residual_is_caught(monkeypatch):
    V, K, T = 6, 1, 1.0
    zt, zd = _dists(V, K, seed=11, sigma=1.5)
    p = ov.softmax(zt[0], T)
    real_max = np.maximum
    # max(0, q - p) instead of max(0, p - q): the replacement law is wrong
    monkeypatch.setattr(ov.np, "maximum", lambda a, b: real_max(a, -b) if np.ndim(b) else real_max(a, b))
    out, _, _ = _trials(zt, zd, T, 20000, seed=5)
    monkeypatch.setattr(ov.np, "maximum", real_max)
    assert chisquare(np.bincount(out[:, 0], minlength=V), p * 20000).pvalue < 1e-6


def test_planted_mistake_ignoring_temperature_is_caught(monkeypatch):
    V, K, T = 4, 2, 0.5
    zt, zd = _dists(V, K, seed=42)
    law = laws.exact_outcome_law(ov.softmax(zt, T), ov.softmax(zd, T))
    real = ov.softmax
    monkeypatch.setattr(ov, "softmax", lambda z, T_: real(z, 1.0))
    out, al, _ = _trials(zt, zd, T, 12000, seed=2)
    monkeypatch.setattr(ov, "softmax", real)
    obs = {}
    for b in range(12000):
        key = tuple(int(v) for v in out[b, :al[b]])
        obs[key] = obs.get(key, 0) + 1
    obs = {k: v for k, v in obs.items() if k in law}
    n = sum(obs.values())
    assert _chi2(obs, law, n) < 1e-6


@pytest.mark.parametrize("T", [0.5, 1.0, 3.0])
def test_softmax_matches_torch_fp64(T):
    """softmax(z / T) (publishertech section 2 "Modified Rejection Sampling":
    p and q are the models' next-token distributions at temperature T)
    against torch.softmax in float64, an independent library routine, on
    logits of several scales and with a large common offset; the oracle's
    form subtracts the maximum first, so it must also be invariant to a
    shift of every logit by the same constant."""
    import torch
    g = np.random.default_rng(int(T * 10))
    for V, scale in ((7, 1.0), (1001, 3.0), (32000, 1.28), (4096, 20.0)):
        z = g.standard_normal((3, V)) * scale
        ref = torch.softmax(torch.from_numpy(z) / T, dim=-1).numpy()
        got = ov.softmax(z, T)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)
        assert np.allclose(got.sum(-1), 1.0, rtol=0, atol=1e-12)
        shifted = ov.softmax(z + 1234.5, T)
        assert np.allclose(shifted, got, rtol=1e-9, atol=1e-300)
    # one dominant logit at a low temperature: nearly one-hot, as torch has it
    z = np.array([0.0, 5.0, 1.0, 5.0 - 1e-3])
    assert np.allclose(ov.softmax(z, 0.01), torch.softmax(torch.from_numpy(z) / 0.01, -1).numpy(),
                       rtol=1e-12, atol=1e-300)
