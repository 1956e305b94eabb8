"""The allocation-free rejection-sampling entry point
(spec_verify_accept_noalloc, static per-device scratch) against
spec_verify_accept (caller workspace) through the C ABI: two calls in a row,
the second smaller, must give bit-identical tokens, acceptance lengths and
p(x), q(x); a greedy call follows.  Both run the same kernels, so any
difference would come from the scratch handling."""
import numpy as np
import torch

import workload
from oracle import verify as ov
from tests.gpu_helpers import cpu, gpu, note, require_gpu

CALLS = [
    # B, K, V, T, scale, sigma, seed, step
    (64, 4, 32000, 1.0, 1.28, 0.38, 11, 0),
    (3, 2, 5000, 0.7, 1.3, 0.5, 12, 4),
    (8, 4, 128256, 0.0, 1.81, 0.54, 13, 1),
]


def _inputs(B, K, V, T, scale, sigma, seed, step):
    t, d = workload.make_synthetic_logits(B, K, V, scale, sigma, seed=seed)
    x = ov.sample_draft_tokens(d, T, seed, step)
    return (torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(), torch.from_numpy(x).cuda())


@gpu
def test_accept_noalloc_matches_workspace_entry_point():
    sv = require_gpu()
    for B, K, V, T, scale, sigma, seed, step in CALLS:
        note(f"no-alloc accept vs accept: B={B} K={K} V={V} T={T}")
        tt, dd, xx = _inputs(B, K, V, T, scale, sigma, seed, step)
        outs = []
        for fn in ("workspace", "noalloc"):
            out = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
            al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
            p_at = torch.full((B, K), -1.0, dtype=torch.float32, device="cuda")
            q_at = torch.full((B, K), -1.0, dtype=torch.float32, device="cuda")
            if fn == "workspace":
                sv.accept(tt, dd, xx, T, seed, step, out_tokens=out, accept_len=al, p_at=p_at,
                          q_at=q_at)
            else:
                sv.accept_noalloc(tt, dd, xx, T, seed, step, out, al, p_at=p_at, q_at=q_at)
            torch.cuda.synchronize()
            outs.append((cpu(out), cpu(al), cpu(p_at), cpu(q_at)))
        (o0, a0, p0, q0), (o1, a1, p1, q1) = outs
        assert np.all((a1 >= 1) & (a1 <= K + 1))
        assert np.array_equal(a0, a1) and np.array_equal(o0, o1)
        if T > 0:
            assert np.array_equal(p0.view(np.uint32), p1.view(np.uint32))
            assert np.array_equal(q0.view(np.uint32), q1.view(np.uint32))
        note(f"  identical: AL {a1[:8].tolist()}")
