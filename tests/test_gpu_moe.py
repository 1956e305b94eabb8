"""GPU parity of the mixture-of-experts verification forward
(include/spec_verify_moe.h) against oracle/moe.py.

Logits within 2e-2 absolute (bf16 inputs, fp32 accumulation), for every row
whose router scores keep the k-th and (k+1)-th expert at least
oracle.moe.ROUTE_BAND apart in every block (closer rows can route
differently under another summation order; they are counted and set aside,
like near-threshold accept decisions).  The number of distinct experts per
block equals the oracle's when no row is set aside.
"""
import numpy as np
import pytest
import torch

import workload
from oracle import moe as om
from tests.gpu_helpers import TOL_BF16, cpu, gpu, note, require_gpu, to_dev_weight


def _device(sv, model, top_k, head="w_head"):
    return sv.MoEModel.packed(to_dev_weight(model["w_router"]), to_dev_weight(model["w_up"]),
                              to_dev_weight(model["w_down"]),
                              torch.from_numpy(model["gain"]).cuda(), to_dev_weight(model[head]), top_k)


def _check(sv, w, model, M, sub):
    m = _device(sv, model, w.top_k)
    h = workload.make_hidden(workload.Workload("h", w.d, 1, 1, 1, "f32", 1, 1, 0, 1, "std_0.02", w.seed),
                             M, sub=sub)
    active = torch.zeros(w.n_layers, dtype=torch.int32, device="cuda")
    z = cpu(m.forward(torch.from_numpy(h).cuda(), active=active))
    ref, gap, used = om.forward(model, h, w.top_k)
    ok = gap >= om.ROUTE_BAND
    err = np.abs(z.astype(np.float64) - ref)[ok]
    note(f"  moe E={w.n_experts} k={w.top_k} M={M}: max |dlogit| {err.max():.3g} over {ok.sum()} rows, "
         f"{(~ok).sum()} near-tie rows set aside; active {cpu(active).tolist()}")
    assert np.all(np.isfinite(z))
    assert err.max() <= TOL_BF16
    if ok.all():
        assert cpu(active).tolist() == [len(u) for u in used]
    return z


@gpu
@pytest.mark.parametrize("M", [1, 5, 9, 12, 16, 17, 64, 65, 100, 300])
def test_small_moe_forward(M):
    sv = require_gpu()
    # several weight fragments, a ragged vocabulary, experts idle and busy
    w = workload.MoEWorkload("moe-small", 256, 160, 16, 4, 2, 1001, 1, 4, 0.3, 1.0, 5)
    model = workload.make_moe_model(w, draft_head=False)
    _check(sv, w, model, M, M)


@gpu
def test_top1_and_all_experts():
    sv = require_gpu()
    for E, k in ((8, 1), (8, 8), (1, 1)):
        w = workload.MoEWorkload("moe-edge", 128, 64, E, k, 2, 333, 1, 4, 0.3, 1.0, 7)
        _check(sv, w, workload.make_moe_model(w, draft_head=False), 33, E * 10 + k)


@gpu
@pytest.mark.parametrize("M", [3, 40])
def test_widest_router(M):
    """256 experts, top-8 (the largest the library takes): every lane of a
    top-k wave holds four experts."""
    sv = require_gpu()
    w = workload.MoEWorkload("moe-wide", 128, 64, 256, 8, 2, 333, 1, 4, 0.3, 1.0, 13)
    _check(sv, w, workload.make_moe_model(w, draft_head=False), M, M + 256)


@gpu
def test_full_size_moe_rows():
    """The 64-expert top-6 stack at its benchmark size, B = 1, K = 4."""
    sv = require_gpu()
    w = workload.MOE_WORKLOADS["moe-64e-top6-b1-k4"]
    model = workload.make_moe_model(w, draft_head=False)
    _check(sv, w, model, w.M, 0)


@gpu
def test_moe_forward_is_deterministic():
    sv = require_gpu()
    w = workload.MoEWorkload("moe-small", 256, 160, 16, 4, 2, 1001, 1, 4, 0.3, 1.0, 5)
    m = _device(sv, workload.make_moe_model(w, draft_head=False), 4)
    h = torch.from_numpy(np.random.default_rng(0).standard_normal((200, 256)).astype(np.float32)).cuda()
    assert torch.equal(m.forward(h), m.forward(h))


@gpu
@pytest.mark.parametrize("M", [4, 7, 100])
def test_exact_router_ties(M):
    """Every expert of a block has the same router row, so all scores tie
    exactly (in fp64 and in the kernel's fp32 alike): ties go to the lower
    id, so experts 0 .. k-1 serve every position with equal weights.  No row
    is set aside here: the rule decides, not the summation order.  M = 4
    routes in one workgroup; M = 7 leaves a ragged top-k workgroup; M = 100
    spans two router row blocks."""
    sv = require_gpu()
    for E, k in ((2, 1), (8, 3)):
        w = workload.MoEWorkload("moe-ties", 128, 64, E, k, 2, 333, 1, 4, 0.3, 1.0, 11)
        model = workload.make_moe_model(w, draft_head=False)
        model["w_router"][:] = model["w_router"][:, :1]
        m = _device(sv, model, k)
        h = workload.make_hidden(workload.Workload("h", w.d, 1, 1, 1, "f32", 1, 1, 0, 1, "std_0.02",
                                                   w.seed), M, sub=E)
        active = torch.zeros(w.n_layers, dtype=torch.int32, device="cuda")
        z = cpu(m.forward(torch.from_numpy(h).cuda(), active=active))
        ref, _, used = om.forward(model, h, k)
        assert [sorted(u) for u in used] == [list(range(k))] * w.n_layers
        err = np.abs(z.astype(np.float64) - ref)
        note(f"  ties E={E} k={k} M={M}: max |dlogit| {err.max():.3g}")
        assert err.max() <= TOL_BF16
        assert cpu(active).tolist() == [k] * w.n_layers
