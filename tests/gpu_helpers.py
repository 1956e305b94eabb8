"""Shared helpers of the GPU parity tests (not a test module).

Inputs come from ``workload`` (seeded); expected values come only from
``oracle``.  Nothing here feeds a GPU result back into the oracle.
"""
from __future__ import annotations

import functools
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import workload
from oracle import forward as oforward, verify as overify

gpu = pytest.mark.gpu


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_step_amd as sv
    sv.lib()            # raises loudly if the library is missing
    return sv


def to_dev_weight(w: np.ndarray) -> torch.Tensor:
    """uint16 bf16 patterns -> torch.bfloat16 on the GPU; fp32 passes through."""
    if w.dtype == np.uint16:
        return torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w)).cuda()


def device_model(sv, model: dict, head: str = "w_head", tiled: bool = False):
    args = (to_dev_weight(model["w_up"]), to_dev_weight(model["w_down"]),
            torch.from_numpy(model["gain"]).cuda(), to_dev_weight(model[head]))
    return sv.Model.packed(*args) if tiled else sv.Model(*args)


def cpu(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def compare_accept(gpu_out, gpu_al, ref_out, ref_al, results, requests=None):
    """Bit-exact comparison of emitted tokens / AL, setting aside requests whose
    oracle run has a decision within the stated band (|u - p/q| < 1e-5, or a
    replacement draw within 1e-5 * R of a CDF boundary).  Returns the number
    of requests set aside."""
    requests = range(len(ref_al)) if requests is None else requests
    near, bad = 0, []
    for b in requests:
        if results[b] is not None and results[b].near:
            near += 1
            continue
        if gpu_al[b] != ref_al[b] or not np.array_equal(gpu_out[b], ref_out[b]):
            bad.append((b, int(gpu_al[b]), int(ref_al[b]), gpu_out[b].tolist(), ref_out[b].tolist()))
    assert not bad, f"{len(bad)} mismatching requests, first: {bad[:3]}"
    return near


def step_band_near(res: overify.RequestResult, eps: float, T: float, zt_rows: np.ndarray) -> bool:
    """Whether an oracle request lies within the band that a logit error of at
    most `eps` (the measured GPU-vs-oracle difference on that request's target
    rows) can move.  The draft logits are identical inputs on both sides, so
    log(p/q) moves by at most 2 eps / T; a CDF position moves by at most
    2 eps / T of total mass; an argmax can flip only when the top two logits
    are within 2 eps."""
    if T == 0.0:
        for j in range(res.accept_len):
            z = np.sort(zt_rows[j])[::-1]
            if len(z) > 1 and z[0] - z[1] <= 2 * eps + 1e-6:
                return True
        return False
    dl = 2 * eps / T + 1e-5
    for d in res.decisions:
        if np.isfinite(d.ratio) and d.ratio > 0 and abs(math.log(d.u) - math.log(d.ratio)) <= dl:
            return True
    if res.draw is not None:
        dr = res.draw
        band = (4 * eps / T + 1e-5) * max(dr.total, 1e-30)
        if min(abs(dr.threshold - dr.c_lo), abs(dr.c_hi - dr.threshold)) <= band:
            return True
    return res.near


def logits_like_scale(w: workload.Workload) -> float:
    """Spread of a normed head's logits: sqrt(d) * std(W_head) (bf16 stacks)."""
    return math.sqrt(w.d) * w.weight_std


TOL_BF16 = 2e-2          # logits, bf16 inputs with fp32 accumulation
TOL_F32 = 1e-4           # logits, fp32 stack

_SPREAD_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                            "bf16_stack_spread.json")


def full_stack_tol(name: str) -> float:
    """Logit tolerance for a full bf16 stack: the stated 2e-2, or 1.5x the
    spread between two valid accumulation orders of the oracle itself on the
    same rows (tests/golden/bf16_stack_spread.json), whichever is larger."""
    with open(_SPREAD_FILE) as f:
        spread = json.load(f)["workloads"]
    if name not in spread:
        return TOL_BF16
    return max(TOL_BF16, 1.5 * spread[name]["max_abs"])


def spread_mean(name: str) -> float:
    with open(_SPREAD_FILE) as f:
        return json.load(f)["workloads"][name]["mean_abs"]


@functools.lru_cache(maxsize=1)
def host_workload(name: str):
    """(model with draft head, hidden) of a named workload; the last one is
    kept so consecutive tests of a workload generate it once."""
    w = workload.WORKLOADS[name]
    note(f"{name}: generating weights")
    return workload.make_model(w), workload.make_hidden(w)
