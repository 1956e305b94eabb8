"""The per-launch timing hooks (spec_verify_profile_begin / _pause / _end) on
the GPU: every launch of a forward is recorded once per profiled forward,
launches made while paused are not, and the summed algorithmic bytes are the
per-launch figures times the launches.  Timing only; the forward's numerics
are covered by the forward parity tests."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import device_model, gpu, host_workload, note, require_gpu


@gpu
def test_profile_counts_launches_and_pause_skips_them():
    sv = require_gpu()
    model, hidden = host_workload("tiny-fp32")
    m = device_model(sv, model)
    hid = torch.from_numpy(np.ascontiguousarray(hidden)).cuda()
    ws = sv.workspace(m.forward_workspace_bytes(hid.shape[0]))
    logits = m.forward(hid, ws=ws)
    torch.cuda.synchronize()
    note("tiny-fp32: one profiled forward")
    sv.profile_begin(256)
    m.forward(hid, logits=logits, ws=ws)
    one = sv.profile_end(64)
    assert one, "a profiled forward recorded no launch"
    for name, (n, ms, b, f) in one.items():
        assert n >= 1 and ms > 0.0 and b >= 0.0 and f >= 0.0, (name, n, ms, b, f)

    note("tiny-fp32: profiled, paused, profiled again")
    sv.profile_begin(256)
    try:
        m.forward(hid, logits=logits, ws=ws)
        sv.profile_pause(True)
        for _ in range(3):
            m.forward(hid, logits=logits, ws=ws)
        sv.profile_pause(False)
        m.forward(hid, logits=logits, ws=ws)
    finally:
        two = sv.profile_end(64)
    torch.cuda.synchronize()
    assert set(two) == set(one)
    for name in one:
        n1, _, b1, f1 = one[name]
        n2, ms2, b2, f2 = two[name]
        assert n2 == 2 * n1, (name, n1, n2)
        assert b2 == pytest.approx(2 * b1) and f2 == pytest.approx(2 * f1), name
        assert ms2 > 0.0

    # the cap: launches past max_launches run untimed
    total = sum(v[0] for v in one.values())
    sv.profile_begin(1)
    m.forward(hid, logits=logits, ws=ws)
    capped = sv.profile_end(64)
    assert sum(v[0] for v in capped.values()) == 1 <= total
    with pytest.raises(RuntimeError):
        sv.profile_pause(True)              # profiling is off again
