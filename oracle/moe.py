"""Verification forward of a mixture-of-experts target (oracle side; test
infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package; the library never does.

Every block of the target is a pre-norm MoE block: a router scores the E
experts for each position, the top_k are kept (ties go to the lower expert
id) and weighted by the softmax of their router scores, and each chosen
expert is a SiLU MLP of the dense block's form; the weighted expert outputs
are added to the residual stream in rank order.  The pages describe the
effect, not the block: verification of more positions activates more
experts, so the weight bytes a step streams grow with B (K + 1) until every
expert is loaded (Cohere, "Dynamic speculative decoding"; NVIDIA co-design
post, "Draft length and performance of linear layers": grouped expert
GEMMs).  Precision follows the dense oracle: bf16 rounding of the norm
output and of the SiLU output, fp64 arithmetic elsewhere.

Pinned by: one expert with top-1 reduces to the dense block; identical
experts reduce to the dense block for any top_k (the weights sum to one);
the routing rule on hand-worked logits (ties, weights, the top-k gap);
top_k = E gives the full softmax; relabelling the experts (router rows and
expert weights together) leaves the logits unchanged.
"""
from __future__ import annotations

import numpy as np

from oracle.forward import RMS_EPS, bf16_round, head, rmsnorm, silu, weights_f64

# rows whose k-th and (k+1)-th router scores are closer than this (in any
# block) can route differently under a different summation order; tests set
# them aside like near-threshold accept decisions
ROUTE_BAND = 1e-4


def route(z: np.ndarray, k: int):
    """Experts chosen for router scores z [E] (rank order, ties to the lower
    id), their softmax weights over the chosen scores, and the gap between
    the k-th and (k+1)-th score (inf when k = E)."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.size), -z))
    sel = order[:k]
    w = np.exp(z[sel] - z[sel].max())
    w /= w.sum()
    gap = z[order[k - 1]] - z[order[k]] if k < z.size else np.inf
    return sel, w, gap


def final_activation(model: dict, hidden: np.ndarray, top_k: int, eps: float = RMS_EPS):
    """a_f [rows, d] (fp64), the smallest router gap of every row over the
    blocks, and the set of experts each block used."""
    h = np.asarray(hidden, dtype=np.float64)
    g = np.asarray(model["gain"], dtype=np.float64)
    L = model["w_router"].shape[0]
    rows = h.shape[0]
    min_gap = np.full(rows, np.inf)
    used = []
    for l in range(L):
        a = bf16_round(rmsnorm(h, g[l], eps))
        z = a @ weights_f64(model["w_router"][l]).T
        cache = {}
        y = np.zeros_like(h)
        used_l = set()
        for r in range(rows):
            sel, w, gap = route(z[r], top_k)
            min_gap[r] = min(min_gap[r], gap)
            for j, e in enumerate(sel):
                e = int(e)
                used_l.add(e)
                if e not in cache:
                    cache[e] = (weights_f64(model["w_up"][l, e]), weights_f64(model["w_down"][l, e]))
                up, down = cache[e]
                s = bf16_round(silu(a[r] @ up.T))
                y[r] += w[j] * (s @ down.T)
        h = h + y
        used.append(used_l)
    return bf16_round(rmsnorm(h, g[L], eps)), min_gap, used


def forward(model: dict, hidden: np.ndarray, top_k: int, heads=("w_head",), eps: float = RMS_EPS):
    """(logits for each requested head, min router gap per row, experts
    used per block)."""
    a_f, gap, used = final_activation(model, hidden, top_k, eps)
    outs = tuple(head(a_f, model[name]) for name in heads)
    return (outs[0] if len(outs) == 1 else outs), gap, used


def expected_active(n_experts: int, top_k: int, rows: int) -> float:
    """Distinct experts a block touches when every row picks top_k of
    n_experts uniformly at random: E (1 - (1 - k/E)^rows)."""
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** rows)
