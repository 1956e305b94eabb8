"""Closed forms and exact laws of the verification step (oracle side).

* ``acceptance_prob``: beta = sum_y min(p(y), q(y)), the chance that a draft
  token drawn from q is accepted (publishertech, section 2 "Proof of
  Distributional Invariance").
* ``al_law``: with independent positions, P(AL = a) = beta_1 ... beta_{a-1}
  (1 - beta_a) for a <= K and P(AL = K + 1) = beta_1 ... beta_K (from the
  same proof and the truncation at the first rejection, mohashari
  "Speculative Decoding Mechanics").
* ``expected_tokens``: E[N] = 1 + sum_{i=1}^{gamma} alpha^i =
  (1 - alpha^(gamma+1)) / (1 - alpha) for a constant acceptance rate
  (publishertech, section 2 "Theoretical Speedup Equation").
* ``speedup``: S = E[N] / (1 + gamma c) (same section).
* ``exact_outcome_law``: the exact probability of every emitted token tuple,
  by enumerating all draft tuples (tiny V and K only).  Used as the law a
  chi-square test compares the sampler against.

Pinned by: the values the pages print for the speedup equation (E[N] about
1.42 at alpha = 0.3, gamma = 5; S = 3.52 for E[N] = 4.4 and c = 0.05; 1.13
and 0.94 for alpha = 0.3 at c = 0.05 / 0.10); the law sums to one; the
marginal of the first emitted token equals p_1 (the invariance proof).
"""
from __future__ import annotations

import itertools

import numpy as np


def acceptance_prob(p: np.ndarray, q: np.ndarray) -> float:
    return float(np.minimum(p, q).sum())


def al_law(betas) -> np.ndarray:
    """P(AL = a) for a = 1..K+1, given per-position acceptance probabilities."""
    betas = list(betas)
    K = len(betas)
    law = np.zeros(K + 1)
    keep = 1.0
    for a in range(1, K + 1):
        law[a - 1] = keep * (1.0 - betas[a - 1])
        keep *= betas[a - 1]
    law[K] = keep
    return law


def expected_al(betas) -> float:
    law = al_law(betas)
    return float(np.dot(np.arange(1, len(law) + 1), law))


def expected_tokens(alpha: float, gamma: int) -> float:
    """E[N] = (1 - alpha^(gamma+1)) / (1 - alpha); gamma + 1 when alpha = 1."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speedup(expected_n: float, gamma: int, c: float) -> float:
    """S = E[N] / (1 + gamma * c)."""
    return expected_n / (1.0 + gamma * c)


def exact_outcome_law(p: np.ndarray, q: np.ndarray) -> dict:
    """Exact law of the emitted tuple for one request.

    p [K+1, V] target distributions (row K is the bonus row), q [K, V] draft
    distributions; draft tokens x_j ~ q_j independently.  Returns
    {tuple(tokens): probability}.  Cost V^K * K * V: tiny inputs only."""
    K1, V = p.shape
    K = K1 - 1
    law: dict = {}

    def add(key, pr):
        if pr > 0.0:
            law[key] = law.get(key, 0.0) + pr

    resid = []
    for j in range(K):
        r = np.maximum(0.0, p[j] - q[j])
        resid.append(r / r.sum() if r.sum() > 0 else p[j])
    for xs in itertools.product(range(V), repeat=K):
        px = float(np.prod([q[j][xs[j]] for j in range(K)])) if K else 1.0
        if px == 0.0:
            continue
        keep = px
        for j in range(K):
            acc = min(1.0, p[j][xs[j]] / q[j][xs[j]])
            for y in range(V):
                add(tuple(xs[:j]) + (y,), keep * (1.0 - acc) * resid[j][y])
            keep *= acc
        for y in range(V):
            add(tuple(xs) + (y,), keep * p[K][y])
    return law
