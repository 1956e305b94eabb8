"""Draft-length choice (oracle side; test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package; the library never does.

* ``choose_k``: for each batch size B, the draft length K with the largest
  goodput = AL(K) / ITL(B, K), ITL = T_verif(B (K + 1)) + T_draft(B, K)
  (Cohere, "Hardware-Aware, Dynamic Speculative Decoding (DSD)", section
  "Dynamic speculative decoding"), T_verif linear between measured row
  counts and unknown outside them; ties go to the smaller K.
* ``speedup_vs_no_draft``: the NVIDIA co-design post's speedup
  T_verif(B) AL / (T_verif(B (1 + D)) + T_draft(B, D)) (section "What is
  speculative decoding?").
* ``window_k``: the dynamic window sizing of mohashari "Speculative
  Decoding in Production", section "Production Failure Modes and Mitigation
  Strategies", item 1 "Draft Acceptance Rate Collapse (Entropy Shift)": the
  reduced window when the mean acceptance length over the last `window`
  requests is below the threshold (1.5 over 10 on the page), else the
  normal one.

Pinned by: the pages' printed speedups (3.52 at E[N] = 4.4, gamma = 5,
c = 0.05; 1.13 / 0.94 at alpha = 0.3) reproduced as goodput ratios with a
flat verification time and a draft cost of gamma c; closed-form optima in
the two limits (flat T_verif and no draft cost: the largest K; T_verif
proportional to rows: K = 0); the DSD page's statement that for a dense
model the optimal K does not increase with the batch size.
"""
from __future__ import annotations

import numpy as np


def verif_time(m_rows, t_verif, M):
    """T_verif at M rows (linear between measured counts), None outside."""
    m = np.asarray(m_rows, dtype=np.float64)
    if M < m[0] or M > m[-1]:
        return None
    return float(np.interp(M, m, np.asarray(t_verif, dtype=np.float64)))


def goodput(m_rows, t_verif, al, B, K, t_draft=0.0):
    t = verif_time(m_rows, t_verif, B * (K + 1))
    if t is None:
        return None
    return al[K] / (t + t_draft)


def choose_k(m_rows, t_verif, al, batch, t_draft=None):
    """Per batch size: (K, goodput) maximising goodput; the first K on ties."""
    out = []
    for i, B in enumerate(batch):
        best = None
        for K in range(len(al)):
            c = 0.0 if t_draft is None else float(t_draft[i][K])
            g = goodput(m_rows, t_verif, al, B, K, c)
            if g is None:
                continue
            if best is None or g > best[1]:
                best = (K, g)
        if best is None:
            raise ValueError(f"no draft length puts batch {B} inside the measured rows")
        out.append(best)
    return out


def speedup_vs_no_draft(t_b, t_bd, al, t_draft):
    """T_verif(B) AL / (T_verif(B (1 + D)) + T_draft(B, D))."""
    return t_b * al / (t_bd + t_draft)


def window_k(accept_len, window, threshold, k_high, k_low):
    valid = [a for a in accept_len if a >= 1]
    recent = valid[-window:] if window > 0 else []
    if len(recent) < window:
        return k_high
    return k_low if float(np.mean(recent)) < threshold else k_high
