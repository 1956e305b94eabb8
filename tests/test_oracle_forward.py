"""Pins for the oracle's target forward (fp64)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workload
from oracle import forward as of


def _torch_forward(model, hidden, bf16):
    """The same block order built from torch library routines in float64."""
    def w(t):
        if t.dtype == np.uint16:
            t = workload.bf16_bits_to_f32(t)
        return torch.from_numpy(np.asarray(t, dtype=np.float64))

    def rnd(x):
        # bf16 rounding through torch's own conversion, applied to the fp32
        # value nearest x (the inputs are built so the fp32 step is exact
        # enough for the tolerance used below)
        return x.to(torch.float32).to(torch.bfloat16).to(torch.float64) if bf16 else x

    g = torch.from_numpy(model["gain"].astype(np.float64))
    h = torch.from_numpy(hidden.astype(np.float64))
    L = model["w_up"].shape[0]
    for l in range(L):
        a = rnd(F.rms_norm(h, (h.shape[-1],), g[l], eps=of.RMS_EPS))
        s = rnd(F.silu(F.linear(a, w(model["w_up"][l]))))
        h = h + F.linear(s, w(model["w_down"][l]))
    a = rnd(F.rms_norm(h, (h.shape[-1],), g[L], eps=of.RMS_EPS))
    return F.linear(a, w(model["w_head"])).numpy()


def _small(wdtype, L=2, d=128, ffn=256, V=512, seed=3):
    wl = workload.Workload("t", d, ffn, L, V, wdtype, 1, 4, 0.3, 1.0,
                           "var_inv_d" if wdtype == "f32" else "std_0.02", seed)
    return wl, workload.make_model(wl), workload.make_hidden(wl, 7)


def test_bf16_round_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000) * 10.0 ** g.integers(-6, 6, 100000),
                        # exact ties between two bf16 values: must go to even
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0])])
    x32 = x.astype(np.float32).astype(np.float64)          # values exactly in fp32
    ref = torch.from_numpy(x32).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(of.bf16_round(x32), ref)
    assert of.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert of.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2 * 2.0 ** -7


def test_rmsnorm_silu_match_torch():
    g = np.random.default_rng(1)
    h = g.standard_normal((5, 64)) * 3
    gain = g.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(gain), eps=1e-5).numpy()
    assert np.allclose(of.rmsnorm(h, gain), ref, rtol=1e-13, atol=1e-13)
    u = g.standard_normal(1000) * 20
    assert np.allclose(of.silu(u), F.silu(torch.from_numpy(u)).numpy(), rtol=1e-13, atol=1e-13)


def test_forward_fp32_matches_torch_composition():
    _, model, hidden = _small("f32")
    ours = of.forward(model, hidden)
    ref = _torch_forward(model, hidden, bf16=False)
    assert np.max(np.abs(ours - ref)) < 1e-10


def test_forward_bf16_matches_torch_composition():
    _, model, hidden = _small("bf16")
    ours = of.forward(model, hidden)
    ref = _torch_forward(model, hidden, bf16=True)
    # the torch side rounds through fp32 first; a handful of activations may
    # land on the other side of a bf16 tie, so compare with a small tolerance
    assert np.max(np.abs(ours - ref)) < 2e-3
    assert np.median(np.abs(ours - ref)) < 1e-6


def test_zero_down_leaves_residual_unchanged():
    _, model, hidden = _small("f32")
    model["w_down"][:] = 0
    ref = of.head(of.rmsnorm(hidden.astype(np.float64), model["gain"][-1]), model["w_head"])
    assert np.allclose(of.forward(model, hidden), ref, rtol=1e-12, atol=1e-12)


def test_zero_layers_is_head_on_normed_input():
    _, model, hidden = _small("f32", L=0)
    a = hidden.astype(np.float64)
    a = a / np.sqrt((a * a).mean(-1, keepdims=True) + 1e-5)
    assert np.allclose(of.forward(model, hidden), a @ model["w_head"].astype(np.float64).T,
                       rtol=1e-12, atol=1e-12)


def test_first_norm_scale_invariance():
    # RMSNorm without eps is invariant to scaling its input; with no blocks
    # the logits depend on the hidden state only through that norm
    _, model, hidden = _small("f32", L=0)
    z1 = of.forward(model, hidden, eps=0.0)
    z2 = of.forward(model, hidden * 1024.0, eps=0.0)   # exact scaling
    assert np.max(np.abs(z1 - z2)) < 1e-12


def test_rows_independent_and_head_blocks():
    _, model, hidden = _small("bf16", V=of._HEAD_ROWS + 37)   # ragged head block
    full = of.forward(model, hidden)
    one = of.forward(model, hidden[3:4])
    assert np.array_equal(full[3:4], one)


def test_draft_head_sigma_zero_equals_target():
    wl = workload.Workload("t", 64, 128, 1, 300, "bf16", 1, 2, 0.0, 1.0, "std_0.02", 5)
    model = workload.make_model(wl, sigma=0.0)
    assert np.array_equal(model["w_head"], model["w_draft_head"])
    hidden = workload.make_hidden(wl)
    zt, zd = of.forward(model, hidden, heads=("w_head", "w_draft_head"))
    assert np.array_equal(zt, zd)


def test_fp32_summation_orders_change_only_rounding():
    """The fp32 evaluation in any summation order stays within fp32 rounding
    of the fp64 reference on an fp32 stack (no bf16 rounding points), and
    different orders really are different rounding sequences."""
    w = workload.WORKLOADS["tiny-fp32"]
    model = workload.make_model(w, draft_head=False)
    h = workload.make_hidden(w, 6, sub=6)
    z64 = of.forward(model, h)
    zs = [of.forward(model, h, accum="f32", k_order=o) for o in (0, 1, 2)]
    for z in zs:
        assert np.abs(z - z64).max() <= 1e-4
    assert not np.array_equal(zs[0], zs[1]) and not np.array_equal(zs[1], zs[2])
    with pytest.raises(ValueError):
        of.forward(model, h, k_order=1)
