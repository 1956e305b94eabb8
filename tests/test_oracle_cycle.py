"""Pins of the speculative-cycle oracle (oracle/cycle.py).

A tiny fp32 target (V = 8) makes every law checkable exactly: the draft
loop, the verification and the token hand-over between cycles are each
compared with a value computed directly from the models' next-token
distributions, not with another run of the same code.
"""
import numpy as np
from scipy.stats import chisquare

import workload
from oracle import cycle as oc
from oracle import forward as of
from oracle.verify import softmax

V = 8


def _pair(sigma=0.8, seed=3):
    w = workload.Workload("cycle-tiny", 16, 32, 2, V, "f32", 1, 4, sigma, 1.0, "var_inv_d", seed)
    model = workload.make_model(w)
    drafter = of.truncated(model, 1)
    drafter["w_head"] = model["w_draft_head"]
    return w, model, drafter, workload.make_embedding(w)


def _next_law(model, table, x, T):
    """Next-token distribution of the model at a position holding token x."""
    return softmax(of.forward(model, oc.embed(table, [x]))[0], T)


def test_drafter_equal_to_target_accepts_every_draft():
    w, model, _, table = _pair()
    cur = workload.make_start_tokens(V, 64, seed=1)
    for T in (1.0, 0.7):
        r = oc.cycle(model, model, table, cur, 4, T, seed=5, step=2)
        assert (r.accept_len == 5).all()
        assert (r.out_tokens[:, :4] == r.draft_tokens).all()


def test_greedy_cycles_reproduce_greedy_decoding():
    """At T = 0 the emitted sequence is the target's greedy continuation,
    whatever the drafter proposes."""
    w, model, drafter, table = _pair(sigma=2.0)
    cur = workload.make_start_tokens(V, 6, seed=2)
    emitted, log = oc.generate(model, drafter, table, cur, 3, 0.0, seed=9, steps=5)
    for b in range(cur.size):
        x, ref = int(cur[b]), []
        for _ in range(len(emitted[b])):
            x = int(np.argmax(of.forward(model, oc.embed(table, [x]))[0]))
            ref.append(x)
        assert emitted[b] == ref
    assert any(r.accept_len.min() < 4 for r in log)      # the drafter was wrong sometimes


def test_first_emitted_token_follows_the_target_law():
    """Distributional invariance over one cycle: many requests from the same
    token, each with its own uniforms, emit their first token with the
    target's next-token law, although the drafter's law differs."""
    w, model, drafter, table = _pair(sigma=1.5)
    x0, n, T = 3, 4000, 1.0
    r = oc.cycle(model, drafter, table, np.full(n, x0, np.int32), 3, T, seed=11, step=0)
    p = _next_law(model, table, x0, T)
    q = _next_law(drafter, table, x0, T)
    assert np.abs(p - q).sum() > 0.2
    counts = np.bincount(r.out_tokens[:, 0], minlength=V)
    assert chisquare(counts, p * n).pvalue > 1e-4


def test_draft_tokens_follow_the_drafter_law():
    w, model, drafter, table = _pair()
    x0, n, T = 5, 4000, 0.7
    x, zq, _ = oc.draft(drafter, table, np.full(n, x0, np.int32), 2, T, seed=4, step=1)
    q1 = _next_law(drafter, table, x0, T)
    assert chisquare(np.bincount(x[:, 0], minlength=V), q1 * n).pvalue > 1e-4
    # the second draft is drawn at the first: its law is sum_y q(y | x0) q(. | y)
    q2 = sum(q1[y] * _next_law(drafter, table, y, T) for y in range(V))
    assert chisquare(np.bincount(x[:, 1], minlength=V), q2 * n).pvalue > 1e-4


def test_k_zero_is_one_draw_from_the_target():
    w, model, _, table = _pair()
    x0, n, T = 1, 4000, 1.0
    r = oc.cycle(model, None, table, np.full(n, x0, np.int32), 0, T, seed=2, step=3)
    assert (r.accept_len == 1).all()
    assert (r.next_cur == r.out_tokens[:, 0]).all()
    p = _next_law(model, table, x0, T)
    assert chisquare(np.bincount(r.out_tokens[:, 0], minlength=V), p * n).pvalue > 1e-4


def test_mean_acceptance_length_matches_the_exact_expectation():
    """K = 2 from a fixed token: E[AL] = 1 + beta(x0) + sum_y min(p, q)(y | x0)
    beta(y), with beta(x) = sum min(p(. | x), q(. | x)) (the pages' E[N] with
    position-dependent acceptance, from the proof of distributional
    invariance: a draft y is accepted with probability min(p, q)(y))."""
    w, model, drafter, table = _pair(sigma=1.0)
    x0, n, T = 6, 6000, 1.0
    r = oc.cycle(model, drafter, table, np.full(n, x0, np.int32), 2, T, seed=8, step=4)
    P = {x: _next_law(model, table, x, T) for x in range(V)}
    Q = {x: _next_law(drafter, table, x, T) for x in range(V)}
    beta = {x: np.minimum(P[x], Q[x]).sum() for x in range(V)}
    m = np.minimum(P[x0], Q[x0])
    expect = 1 + beta[x0] + sum(m[y] * beta[y] for y in range(V))
    se = r.accept_len.std() / np.sqrt(n)
    assert abs(r.accept_len.mean() - expect) < 4 * se


def test_next_token_is_the_last_emitted_and_embeddings_pad_with_zeros():
    w, model, drafter, table = _pair()
    cur = workload.make_start_tokens(V, 32, seed=7)
    r = oc.cycle(model, drafter, table, cur, 4, 1.0, seed=1, step=0)
    for b in range(cur.size):
        assert r.next_cur[b] == r.out_tokens[b, r.accept_len[b] - 1]
    e = oc.embed(table, [0, V, -1, 2])
    assert (e[1] == 0).all() and (e[2] == 0).all() and (e[3] == table[2]).all()
