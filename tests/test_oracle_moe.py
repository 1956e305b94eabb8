"""Pins of the MoE oracle (oracle/moe.py)."""
import numpy as np
import pytest

import workload
from oracle import forward as of, moe as om


def _small(E, k, L=2, d=64, f=48, V=101, seed=0):
    w = workload.MoEWorkload("moe-test", d, f, E, k, L, V, 1, 4, 0.3, 1.0, seed)
    return w, workload.make_moe_model(w, draft_head=False)


def _dense_from_expert(model, e):
    return {"w_up": np.ascontiguousarray(model["w_up"][:, e]),
            "w_down": np.ascontiguousarray(model["w_down"][:, e]),
            "gain": model["gain"], "w_head": model["w_head"]}


def test_single_expert_top1_is_the_dense_block():
    w, model = _small(1, 1)
    h = np.random.default_rng(1).standard_normal((7, w.d))
    z, gap, used = om.forward(model, h, 1)
    ref = of.forward(_dense_from_expert(model, 0), h)
    assert np.allclose(z, ref, rtol=0, atol=1e-12)
    assert np.all(np.isinf(gap)) and used == [{0}, {0}]


def test_identical_experts_reduce_to_dense_for_any_top_k():
    w, model = _small(8, 3)
    model["w_up"][:] = model["w_up"][:, :1]
    model["w_down"][:] = model["w_down"][:, :1]
    h = np.random.default_rng(2).standard_normal((5, w.d))
    z, _, _ = om.forward(model, h, 3)
    assert np.allclose(z, of.forward(_dense_from_expert(model, 0), h), rtol=0, atol=1e-10)


def test_routing_rule_by_hand():
    z = np.array([0.1, 2.0, 2.0, -1.0, 0.5])
    sel, w, gap = om.route(z, 2)
    assert sel.tolist() == [1, 2] and np.allclose(w, [0.5, 0.5]) and gap == pytest.approx(1.5)
    sel, w, gap = om.route(z, 3)
    e = np.exp(np.array([2.0, 2.0, 0.5]) - 2.0)
    assert sel.tolist() == [1, 2, 4] and np.allclose(w, e / e.sum()) and gap == pytest.approx(0.4)
    sel, w, gap = om.route(z, 5)
    full = np.exp(z - z.max())
    assert sel.tolist() == [1, 2, 4, 0, 3] and np.allclose(w, full[sel] / full.sum())
    assert np.isinf(gap)


def test_relabelled_experts_give_the_same_logits():
    w, model = _small(6, 2)
    h = np.random.default_rng(3).standard_normal((6, w.d))
    z, gap, used = om.forward(model, h, 2)
    perm = np.random.default_rng(4).permutation(6)       # new id of old expert e is perm[e]
    m2 = dict(model)
    for key in ("w_router", "w_up", "w_down"):
        arr = np.empty_like(model[key])
        arr[:, perm] = model[key]
        m2[key] = arr
    z2, gap2, used2 = om.forward(m2, h, 2)
    assert np.allclose(z2, z, rtol=0, atol=1e-12) and np.allclose(gap2, gap)
    assert used2 == [{int(perm[e]) for e in u} for u in used]


def test_expected_active_limits():
    assert om.expected_active(64, 6, 1) == pytest.approx(6.0)
    assert om.expected_active(64, 6, 10_000) == pytest.approx(64.0)
