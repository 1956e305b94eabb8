"""Oracle modified rejection sampling for one verification step (fp64).

The rule, as the pages state it:

* target distribution p and draft distribution q per drafted position;
  accept draft token x with probability min(1, p(x)/q(x)), i.e. draw
  u ~ U(0, 1) and accept iff u <= p(x)/q(x) (publishertech, section 2
  "Modified Rejection Sampling"; mohashari "Speculative Decoding
  Mechanics: The Mathematics of Verification"; klu.ai "Mathematical
  Guarantee");
* on the first rejection, discard that token and every later draft and emit
  one token from p'(x) = max(0, p(x) - q(x)) / sum_y max(0, p(y) - q(y))
  (same sections);
* if every draft is accepted, the target still emits one more token from its
  own distribution at the next position, so the number of tokens produced
  per step (the acceptance length AL) lies in [1, 1 + K] (NVIDIA co-design
  post, section "What is speculative decoding?");
* at temperature 0 (greedy) verification keeps the longest prefix of drafts
  that equal the target's argmax and then emits the target's argmax, which is
  the output of plain greedy decoding (same section; klu.ai "Mathematical
  Guarantee").

Readings where the pages are silent:

* K + 1 target rows per request: row j (0-based) holds p for draft token j,
  row K the bonus distribution.
* temperature T > 0 divides both target and draft logits; p = softmax(z/T)
  computed as exp((z - max z)/T) / sum.  No top-k / top-p.
* u for the accept test is U_acc(b, j) in (0, 1]; the replacement uses
  u' = U_res(b, j) in [0, 1) and inverse-CDF order over ascending token ids:
  y* = min{y : C_y > u' * R} with C the running sum of the weights and R their
  total.  If rounding leaves no such y, the last token with positive weight
  is taken.  If R = 0 after a rejection (impossible in exact arithmetic) the
  replacement is drawn from p by the same rule.
* accept iff u <= p/q in IEEE arithmetic: q = 0 < p accepts (ratio +inf),
  p = q = 0 rejects (ratio NaN).
* a draft token outside [0, V) marks the whole request invalid: AL = 0 and
  every output slot is -1.
* outputs: tokens [K+1] padded with -1 after AL; AL counts emitted tokens.

Each decision also reports its margin to the nearest threshold so callers can
set aside decisions that lie within a stated band.

Pinned by: AL in [1, K+1]; p = q gives AL = K + 1 for every seed;
disjoint supports give AL = 1; greedy equals a textbook greedy loop;
the exact law of (AL, tokens) from ``laws.exact_outcome_law`` (chi-square);
the emitted token's marginal equals p (the invariance proof, publishertech
section 2 "Proof of Distributional Invariance"); acceptance frequency equals
sum_y min(p, q); mean AL equals the closed form (publishertech section 2
"Theoretical Speedup Equation").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import philox

ACCEPT_BAND = 1e-5      # |u - p/q| below this: decision is near-threshold
RESAMPLE_BAND = 1e-5    # |u' R - C| below this * R: draw is near a CDF boundary


@dataclass
class Decision:
    j: int                 # 1-based draft position
    u: float
    ratio: float
    accepted: bool
    near: bool


@dataclass
class Draw:
    j: int                 # 1-based position the token is emitted for
    token: int
    threshold: float       # u' * R
    c_lo: float            # C_{y*-1} (0 if y* is the first positive weight)
    c_hi: float            # C_{y*}
    total: float           # R
    near: bool
    fallback: bool = False  # R == 0 after rejection: drawn from p instead


@dataclass
class RequestResult:
    tokens: np.ndarray                 # [K+1] int32, -1 padded
    accept_len: int
    decisions: list = field(default_factory=list)
    draw: Draw | None = None

    @property
    def near(self) -> bool:
        return any(d.near for d in self.decisions) or (self.draw is not None and self.draw.near)


def softmax(z: np.ndarray, T: float) -> np.ndarray:
    """softmax(z / T) over the last axis: exp((z - max z)/T) / sum."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp((z - z.max(axis=-1, keepdims=True)) / T)
    return e / e.sum(axis=-1, keepdims=True)


def inverse_cdf(w: np.ndarray, u: float):
    """min{y : C_y > u * R} over non-negative weights w (ascending ids).
    Returns (y, threshold, C_{y-1}, C_y, R)."""
    c = np.cumsum(w)
    R = float(c[-1])
    t = u * R
    hit = np.nonzero(c > t)[0]
    if hit.size:
        y = int(hit[0])
    else:
        y = int(np.nonzero(w > 0)[0][-1])
    c_lo = float(c[y - 1]) if y > 0 else 0.0
    return y, t, c_lo, float(c[y]), R


def _draw(j: int, w: np.ndarray, u: float, fallback: bool = False) -> Draw:
    y, t, c_lo, c_hi, R = inverse_cdf(w, u)
    near = min(abs(t - c_lo), abs(c_hi - t)) < RESAMPLE_BAND * R
    return Draw(j, y, t, c_lo, c_hi, R, near, fallback)


def verify_request(zt: np.ndarray, zd: np.ndarray, x: np.ndarray, T: float,
                   seed: int, step: int, b: int) -> RequestResult:
    """One request: zt [K+1, V] target logits, zd [K, V] draft logits,
    x [K] draft tokens.  Returns the emitted tokens and diagnostics."""
    K, V = len(x), zt.shape[-1]
    out = np.full(K + 1, -1, dtype=np.int32)
    if np.any((x < 0) | (x >= V)):
        return RequestResult(out, 0)

    if T == 0.0:
        for j in range(1, K + 1):
            top = int(np.argmax(zt[j - 1]))           # first index of the max
            if int(x[j - 1]) == top:
                out[j - 1] = top
                continue
            out[j - 1] = top
            return RequestResult(out, j)
        out[K] = int(np.argmax(zt[K]))
        return RequestResult(out, K + 1)

    decisions = []
    for j in range(1, K + 1):
        p = softmax(zt[j - 1], T)
        q = softmax(zd[j - 1], T)
        xj = int(x[j - 1])
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = float(np.float64(p[xj]) / np.float64(q[xj]))
        u = float(philox.u_accept(philox.word(b, j, philox.DRAW_ACCEPT, step, seed)))
        accepted = bool(u <= ratio)
        near = bool(abs(u - ratio) < ACCEPT_BAND) if np.isfinite(ratio) else False
        decisions.append(Decision(j, u, ratio, accepted, near))
        if accepted:
            out[j - 1] = xj
            continue
        r = np.maximum(0.0, p - q)
        u2 = float(philox.u_resample(philox.word(b, j, philox.DRAW_RESAMPLE, step, seed)))
        if r.sum() > 0.0:
            d = _draw(j, r, u2)
        else:
            d = _draw(j, p, u2, fallback=True)
        out[j - 1] = d.token
        return RequestResult(out, j, decisions, d)

    p = softmax(zt[K], T)
    u2 = float(philox.u_resample(philox.word(b, K + 1, philox.DRAW_RESAMPLE, step, seed)))
    d = _draw(K + 1, p, u2)
    out[K] = d.token
    return RequestResult(out, K + 1, decisions, d)


def verify(target_logits: np.ndarray, draft_logits: np.ndarray, draft_tokens: np.ndarray,
           T: float, seed: int, step: int, requests=None):
    """Batch form.  target_logits [B, K+1, V], draft_logits [B, K, V],
    draft_tokens [B, K].  ``requests`` restricts the work to some b (the
    others are left as -1 / AL 0 and reported as None).

    Returns (out_tokens [B, K+1] int32, accept_len [B] int32, results list)."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    draft_tokens = np.asarray(draft_tokens).reshape(B, K)
    if K == 0:
        draft_logits = np.zeros((B, 0, V))
    out = np.full((B, K + 1), -1, dtype=np.int32)
    al = np.zeros(B, dtype=np.int32)
    results = [None] * B
    for b in (range(B) if requests is None else requests):
        r = verify_request(target_logits[b], draft_logits[b], draft_tokens[b], T, seed, step, b)
        out[b], al[b], results[b] = r.tokens, r.accept_len, r
    return out, al, results


def sample_draft_tokens(draft_logits: np.ndarray, T: float, seed: int, step: int) -> np.ndarray:
    """Synthetic draft tokens: x[b, j] ~ softmax(draft_logits[b, j] / T) with
    u = U_res(b, j+1, draw 2) and the same inverse-CDF rule; argmax at T = 0.
    (The draft phase is not part of the verification step; this only makes
    inputs whose tokens really come from q.)"""
    B, K, V = draft_logits.shape
    x = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for j in range(K):
            if T == 0.0:
                x[b, j] = int(np.argmax(draft_logits[b, j]))
            else:
                u = float(philox.u_resample(philox.word(b, j + 1, philox.DRAW_DRAFT, step, seed)))
                x[b, j] = inverse_cdf(softmax(draft_logits[b, j], T), u)[0]
    return x
