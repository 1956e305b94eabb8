"""Philox4x32-10 and the uniform draws of the verification step (oracle side).

The pages only ask for "a uniform random value u ~ Uniform(0, 1)" per
decision (publishertech "Speculative Decoding in Large Language Models",
section 2 "Modified Rejection Sampling").  To make every decision
reproducible and independent of launch shape, each draw is one Philox
block keyed by the run's seed and counted by (request, position, draw, step).

Philox4x32 follows Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
As Easy as 1, 2, 3" (SC'11): a 4-word counter and 2-word key; each round
multiplies words 0 and 2 by two fixed 32-bit constants, takes the high and
low halves, and mixes them with words 1 and 3 and the round key; the key is
advanced by the two Weyl constants (golden ratio and sqrt(3) - 1, scaled to
32 bits) between rounds; ten rounds.

Pinned by: the rocRAND Philox4x32-10 engine (compiled from its public
header on the host) for random seeds and counters, and by exact checks of
the two conversions at the end words 0 and 2^32 - 1.
"""
from __future__ import annotations

import numpy as np

MULT0 = 0xD2511F53
MULT1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9   # floor(2^32 / golden ratio)
WEYL1 = 0xBB67AE85   # floor(2^32 * (sqrt(3) - 1))
ROUNDS = 10
_MASK = np.uint64(0xFFFFFFFF)

# Draw ids used by the verification step (third counter word).
DRAW_ACCEPT = 0     # u for "u <= p/q" at draft position j
DRAW_RESAMPLE = 1   # u' for the residual / bonus token
DRAW_DRAFT = 2      # used only to make synthetic draft tokens


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counter words c0..c3 and key words k0, k1
    are integers (or integer arrays that broadcast); returns the four output
    words as uint64 arrays holding 32-bit values."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK for c in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for r in range(ROUNDS):
        if r:
            k0 = (k0 + np.uint64(WEYL0)) & _MASK
            k1 = (k1 + np.uint64(WEYL1)) & _MASK
        prod0 = np.uint64(MULT0) * c0          # < 2^64: exact in uint64
        prod1 = np.uint64(MULT1) * c2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & _MASK
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def word(b, j, draw, step, seed):
    """Output word 0 of Philox at counter (b, j, draw, step), key = seed split
    into its low and high 32-bit halves."""
    seed = int(seed)
    return philox4x32_10(b, j, draw, step, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)[0]


def u_accept(w):
    """Acceptance uniform in (0, 1]: ((w >> 8) + 1) / 2^24.  Exact in fp32
    and fp64; u = 1 is possible, u = 0 is not, so p(x) = 0 never accepts."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(8)) + np.uint64(1)).astype(np.float64) * 2.0 ** -24


def u_resample(w):
    """Resampling uniform in [0, 1): (w >> 8) / 2^24.  Exact in fp32 and fp64."""
    w = np.asarray(w, dtype=np.uint64)
    return (w >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
