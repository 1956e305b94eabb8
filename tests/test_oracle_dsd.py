"""Pins of the draft-length oracle (oracle/dsd.py) against what the pages fix."""
import json
import math
import os

import numpy as np
import pytest

from oracle import dsd, laws

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "speedup_examples.json")


def _trunc2(x):
    return math.floor(x * 100 + 1e-9) / 100


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["speedup"])
def test_printed_speedups_as_goodput_ratios(case):
    """publishertech section 2: S = E[N] / (1 + gamma c) is the goodput ratio
    of K = gamma against K = 0 when the verification time does not change
    with the row count (memory-bound) and drafting costs c per token."""
    gamma, c = case["gamma"], case["c"]
    al = np.ones(gamma + 1)
    al[gamma] = case["expected_n"]
    m_rows, t = [1, 4096], [1.0, 1.0]
    g0 = dsd.goodput(m_rows, t, al, 1, 0, 0.0)
    gk = dsd.goodput(m_rows, t, al, 1, gamma, gamma * c)
    ratio = gk / g0
    want = case["printed"]
    got = round(ratio, 2) if case["rounding"].startswith("exact") else _trunc2(ratio)
    assert got == pytest.approx(want, abs=1e-9)
    # the NVIDIA co-design post's speedup is the same ratio
    assert dsd.speedup_vs_no_draft(1.0, 1.0, case["expected_n"], gamma * c) == pytest.approx(ratio)


def test_flat_verification_without_draft_cost_takes_the_longest_draft():
    """Memory-bound limit (NVIDIA post, 'Selecting the optimal draft length':
    increase D while T_verif stays constant): with AL increasing in K the
    best draft is the longest one, for every batch size."""
    al = [laws.expected_tokens(0.7, k) for k in range(9)]
    res = dsd.choose_k([1, 10_000], [2.0, 2.0], al, [1, 4, 16, 64, 256])
    assert [k for k, _ in res] == [8] * 5


def test_verification_proportional_to_rows_takes_no_draft():
    """Compute-bound limit: T_verif(M) = M makes goodput AL(K) / (B (K+1)),
    which is largest at K = 0 because AL(K) < K + 1 for alpha < 1."""
    al = [laws.expected_tokens(0.9, k) for k in range(9)]
    m = list(range(1, 600))
    res = dsd.choose_k(m, [float(x) for x in m], al, [1, 3, 7, 50])
    assert [k for k, _ in res] == [0, 0, 0, 0]


def test_dense_optimum_does_not_grow_with_batch():
    """Cohere DSD page: for a dense model the optimal K decreases
    monotonically as the batch grows (roofline-shaped T_verif)."""
    ridge = 300.0
    m = list(range(1, 4097))
    t = [max(1.0, x / ridge) + 0.02 * x / ridge for x in m]
    for alpha in (0.5, 0.75, 0.9):
        al = [laws.expected_tokens(alpha, k) for k in range(9)]
        ks = [k for k, _ in dsd.choose_k(m, t, al, [1, 2, 4, 8, 16, 32, 64, 128, 256, 448])]
        assert all(a >= b for a, b in zip(ks, ks[1:])), ks
        assert ks[0] == 8 and ks[-1] == 0


def test_interpolation_and_range():
    m, t = [4, 8, 16], [1.0, 2.0, 6.0]
    assert dsd.verif_time(m, t, 4) == 1.0
    assert dsd.verif_time(m, t, 6) == pytest.approx(1.5)
    assert dsd.verif_time(m, t, 12) == pytest.approx(4.0)
    assert dsd.verif_time(m, t, 3) is None and dsd.verif_time(m, t, 17) is None
    # B = 4 can only use K in {0, 1, 3}; B = 5 only K in {0, 2}
    res = dsd.choose_k(m, t, [1.0, 1.9, 2.5, 3.2], [4, 5])
    assert res[0][0] in (0, 1, 3) and res[1][0] in (0, 2)


def test_ties_go_to_the_shorter_draft():
    res = dsd.choose_k([1, 100], [1.0, 1.0], [1.0, 1.0, 1.0], [2])
    assert res[0][0] == 0


@pytest.mark.parametrize("history,expect", [
    ([1] * 10, 2),                      # mean 1.0 < 1.5: reduced window
    ([2, 1] * 5, 5),                    # mean 1.5 is not below 1.5
    ([3] * 5 + [1] * 10, 2),            # only the last 10 count
    ([1] * 9, 5),                       # not enough history yet
    ([1] * 9 + [0, 0, 1], 2),           # invalid (0) entries are skipped
])
def test_window_rule(history, expect):
    """mohashari "Speculative Decoding in Production", "Production Failure
    Modes and Mitigation Strategies", item 1 "Draft Acceptance Rate Collapse
    (Entropy Shift)": below 1.5 over the last 10 requests the window drops
    from 5 to a small value."""
    assert dsd.window_k(history, 10, 1.5, 5, 2) == expect
