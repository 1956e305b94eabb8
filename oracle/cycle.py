"""The speculative cycle around the verification step (oracle side; test
infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package; the library never does.

One cycle (publishertech, section 1 "The Speculative Cycle: Draft, Verify,
and Accept"): the drafter runs gamma = K steps autoregressively from the
current token, each step drawing the next token from its own distribution
q; the target then scores the current token and the K drafts in one pass and
the modified rejection sampling of ``oracle.verify`` emits AL tokens; the
last emitted token is the next cycle's current token.  K = 0 is plain
decoding (one target pass, one token drawn from p).

Inputs are tokens: the input row of a position holding token x is
``table[x]``.  The drafter in the measurements is an early exit of the target
(its first blocks, its final norm and a head), built by
``oracle.forward.truncated``.

A draft token is drawn like the verification's bonus token: the smallest id
whose running sum of softmax(z / T) exceeds u times the total, with
u = U_res(b, j, 2, step) for draft slot j (Philox draw 2); argmax (lowest
id) at T = 0.

Pinned by (tests/test_oracle_cycle.py), on a tiny target whose next-token
laws are computed directly: a drafter equal to the target accepts every
draft; at T = 0 the emitted tokens are plain greedy decoding of the target
whatever the drafter; the first emitted token follows the target's law
whatever the drafter (chi-squared over requests); the first and second
draft tokens follow the drafter's one- and two-step laws; K = 0 is one draw
from p; the mean acceptance length from a fixed token equals its exact
expectation (the pages' E[N] with acceptance depending on the token).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import philox
from oracle.forward import forward
from oracle.verify import RESAMPLE_BAND, inverse_cdf, softmax, verify


def embed(table: np.ndarray, tokens) -> np.ndarray:
    """Input rows [n, d] (fp64) of the tokens; zero rows outside [0, V)."""
    table = np.asarray(table, dtype=np.float64)
    tokens = np.asarray(tokens).reshape(-1)
    ok = (tokens >= 0) & (tokens < table.shape[0])
    out = np.zeros((tokens.size, table.shape[1]))
    out[ok] = table[tokens[ok]]
    return out


@dataclass
class DraftDraw:
    token: int
    margin: float     # distance of u R to the nearer CDF boundary, over R; at
                      # T = 0 the gap between the two largest logits
    near: bool        # margin below the resample band (T > 0)


def draw_token(z: np.ndarray, T: float, b: int, slot: int, seed: int, step: int) -> DraftDraw:
    """The token drawn for draft slot ``slot`` of request b from logits z."""
    z = np.asarray(z, dtype=np.float64)
    if T == 0.0:
        top = np.sort(z)[::-1]
        return DraftDraw(int(np.argmax(z)), float(top[0] - top[1]) if z.size > 1 else np.inf, False)
    u = float(philox.u_resample(philox.word(b, slot, philox.DRAW_DRAFT, step, seed)))
    y, t, c_lo, c_hi, R = inverse_cdf(softmax(z, T), u)
    margin = min(abs(t - c_lo), abs(c_hi - t)) / R
    return DraftDraw(y, margin, bool(margin < RESAMPLE_BAND))


def draft(drafter: dict, table: np.ndarray, cur, K: int, T: float, seed: int, step: int):
    """The draft loop from the current tokens cur [B]: K steps, each on the
    token the step before drew.  Returns (draft_tokens [B, K] int32,
    draft_logits [B, K, V] fp64, draws: B lists of K DraftDraw)."""
    cur = np.asarray(cur, dtype=np.int64)
    B = cur.size
    V = drafter["w_head"].shape[0]
    x = np.zeros((B, K), dtype=np.int32)
    zq = np.zeros((B, K, V))
    draws = [[] for _ in range(B)]
    tok = cur.copy()
    for j in range(1, K + 1):
        z = forward(drafter, embed(table, tok))
        zq[:, j - 1] = z
        for b in range(B):
            d = draw_token(z[b], T, b, j, seed, step)
            x[b, j - 1] = d.token
            draws[b].append(d)
        tok = x[:, j - 1].astype(np.int64)
    return x, zq, draws


@dataclass
class CycleResult:
    out_tokens: np.ndarray     # [B, K+1] int32, -1 after AL
    accept_len: np.ndarray     # [B] int32
    next_cur: np.ndarray       # [B] int32: the last token emitted
    draft_tokens: np.ndarray   # [B, K]
    draft_logits: np.ndarray   # [B, K, V]
    target_logits: np.ndarray  # [B, K+1, V]
    results: list              # oracle.verify per-request diagnostics
    draft_draws: list          # B lists of K DraftDraw


def cycle(target: dict, drafter: dict | None, table: np.ndarray, cur, K: int, T: float,
          seed: int, step: int) -> CycleResult:
    """One speculative cycle of B requests (drafter unused when K = 0)."""
    cur = np.asarray(cur, dtype=np.int32)
    B = cur.size
    V = target["w_head"].shape[0]
    if K > 0:
        x, zq, draws = draft(drafter, table, cur, K, T, seed, step)
    else:
        x, zq, draws = np.zeros((B, 0), np.int32), np.zeros((B, 0, V)), [[] for _ in range(B)]
    toks = np.concatenate([cur[:, None], x], axis=1)
    zt = forward(target, embed(table, toks)).reshape(B, K + 1, V)
    out, al, res = verify(zt, zq, x, T, seed, step)
    nxt = cur.copy()
    ok = al >= 1
    nxt[ok] = out[np.nonzero(ok)[0], al[ok] - 1]
    return CycleResult(out, al, nxt, x, zq, zt, res, draws)


def generate(target: dict, drafter: dict | None, table: np.ndarray, cur, K: int, T: float,
             seed: int, steps: int, step0: int = 0):
    """Run ``steps`` cycles (step counters step0, step0 + 1, ...); returns
    the emitted tokens of every request (a list per request) and the
    per-cycle results."""
    cur = np.asarray(cur, dtype=np.int32)
    emitted = [[] for _ in range(cur.size)]
    log = []
    for s in range(steps):
        r = cycle(target, drafter, table, cur, K, T, seed, step0 + s)
        for b in range(cur.size):
            emitted[b].extend(int(t) for t in r.out_tokens[b, :r.accept_len[b]])
        cur = r.next_cur
        log.append(r)
    return emitted, log
