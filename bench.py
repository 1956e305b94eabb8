#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verification step on one MI355X.

One step = spec_verify_step over one batch: the target forward over all
B*(K+1) positions (weights streamed once) plus rejection sampling.  Inputs
(weights, hidden states, draft logits, draft tokens) are synthetic and
resident in HBM before timing starts.  The steps are launched eagerly,
back to back on one stream (measured faster than HIP graph replay on this
stack: about 1 us per graph node); the graph-replay time is reported too.

Prints ONE JSON line.  Default (headline) workload: the large-batch step,
B=256, K=2 (d=4096, ffn=14336, L=8, V=128256, bf16, sigma=0.5, T=0.7), the
largest single-GPU configuration; the same line carries nested records
("workloads") of the 70B-layer share (B=8, K=4) and the 8B-shaped step
(B=1, K=4), each with its own roofline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--graph]
                    [--no-cpu-baseline] [--no-nested] [--sweep]

``--sweep`` instead prints one JSON line per (B, K, sigma) point of the
8B-shaped stack (B in 1,4,16,64; K in 1,2,4,8).  ``--crossover`` prints the
forward-only time of each MFMA kernel family (weights streamed to registers
vs LDS-staged GEMM) per row count, to locate the HBM -> MFMA crossover in
B*(K+1).  ``--k-table`` measures T_verif(M) and AL(K) and prints the
goodput-optimal draft length per batch size; ``--attention`` times the paged
attention of the verified positions; ``--moe`` sweeps the mixture-of-experts
target over B x K; ``--cycle`` times whole speculative cycles (draft loop +
verification) against plain decoding.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload  # noqa: E402

METRIC = "verified positions/sec + accepted tokens/sec vs B,K; % HBM / % MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16
VALU_F32_PEAK_TFS = 157.3
# the headline: the largest single-GPU configuration (B=256, K=2, M=768); the
# line also carries these workloads as nested records
HEADLINE = "large-batch-b256-k2"
NESTED = ("70b-layer-share-b8-k4", "8b-shaped-b1-k4")
NESTED_KEYS = ("config", "ms_per_step", "accepted_tokens_per_s", "mean_accept_len",
               "accept_len_hist", "step_ms_p10_p50_p90", "step_hbm_frac", "step_mfma_frac",
               "roofline_step_ms", "forward_ms", "forward_hbm_frac", "forward_mfma_frac",
               "accept_ms", "graph_ms_per_step", "eager_ms_per_step", "roofline", "kernels")
# row counts B*(K+1) of the crossover scan (the sweep's B x K grid spans 2..576)
CROSSOVER_ROWS = (16, 32, 48, 64, 80, 96, 128, 144, 192, 256, 320, 384, 512, 576, 768)


def roofline_time_s(bytes_, flops, bw=HBM_PEAK_GBS * 1e9, peak=MFMA_BF16_PEAK_TFS * 1e12):
    """Lower bound on a step's time: max(bytes / bandwidth, flops / peak)."""
    return max(bytes_ / bw, flops / peak)


def step_work(w: workload.Workload, B: int, K: int, T: float):
    """Algorithmic bytes and flops of one verification step.

    bytes: weights once + hidden in + logits written once and read once +
    draft logits read once + up to two vocab rows per request for the
    replacement draw; flops: 2 * M * (weights' multiply-adds)."""
    M = B * (K + 1)
    es = 2 if w.wdtype == "bf16" else 4
    weights = w.weight_elems() * es + (w.n_layers + 1) * w.d * 4
    logits = M * w.vocab * 4
    draft = 0 if T == 0 else B * K * w.vocab * 4
    resid = 0 if T == 0 else B * 2 * w.vocab * 4
    bytes_ = weights + M * w.d * 4 + 2 * logits + draft + resid
    flops = 2.0 * M * w.weight_elems()
    return bytes_, flops


def measured_traffic(workload_name: str, kernel_label: str):
    """HBM bytes per launch of `kernel_label` from the committed counter
    summary (profiles/hbm_traffic_*.md: FETCH_SIZE and WRITE_SIZE, scaled by a
    plain copy of known size), or None if there is none for this workload or
    the kernel sources changed since the counters were taken."""
    import glob
    import hashlib
    import re
    pkg = os.path.join(ROOT, "speculative_decoding_verification_step_amd")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))):
        m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("workload") != workload_name or kernel_label not in rec["hbm_bytes_per_launch"]:
            continue
        src = b"".join(open(os.path.join(pkg, f), "rb").read() for f in rec["kernel_sources"])
        if hashlib.sha256(src).hexdigest() != rec["kernel_sources_sha256"]:
            return None
        return rec["hbm_bytes_per_launch"][kernel_label]
    return None


def _draft_tokens(zq, T, seed):
    """Draft tokens drawn from q = softmax(zq / T) (Gumbel-max), argmax at T = 0."""
    import torch
    if T == 0:
        return zq.argmax(-1).to(torch.int32).contiguous()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    u = torch.rand(zq.shape, generator=gen, device="cuda").clamp_(1e-20, 1.0)
    return (zq / T - torch.log(-torch.log(u))).argmax(-1).to(torch.int32).contiguous()


_MODEL_CACHE: dict = {}


def _device_models(w, sigma):
    """Target model (packed once per process) and the drafter for `sigma`
    (same blocks, head W_head + sigma * E)."""
    import torch
    import speculative_decoding_verification_step_amd as sv

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    key = (w.name, sigma)
    if _MODEL_CACHE.get("key") != key:
        _MODEL_CACHE.clear()
        torch.cuda.empty_cache()
        model = workload.make_model(w, sigma=sigma)
        d_up, d_down, d_gain = dev(model["w_up"]), dev(model["w_down"]), dev(model["gain"])
        d_head, d_dhead = dev(model["w_head"]), dev(model["w_draft_head"])
        host = {k: model[k] for k in ("w_up", "w_down", "gain", "w_head")}
        del model
        if w.wdtype == "bf16":
            # the weights are packed once, at load time, into the tiled layout
            target = sv.Model.packed(d_up, d_down, d_gain, d_head)
            drafter = sv.Model.packed(d_up, d_down, d_gain, d_dhead)
            del d_up, d_down
        else:
            target = sv.Model(d_up, d_down, d_gain, d_head)
            drafter = sv.Model(d_up, d_down, d_gain, d_dhead)
        _MODEL_CACHE.update(key=key, target=target, drafter=drafter, host=host)
    return _MODEL_CACHE["target"], _MODEL_CACHE["drafter"], _MODEL_CACHE["host"]


def _device_inputs(w, B, K, T, sigma, seed=0):
    import torch
    target, drafter, host = _device_models(w, sigma)
    M = B * (K + 1)
    h = workload.make_hidden(w, M)
    hidden = torch.from_numpy(h).cuda()
    # draft logits: the draft head reads the target's own final hidden state
    zq = drafter.forward(hidden).view(B, K + 1, w.vocab)[:, :K].contiguous()
    x = _draft_tokens(zq, T, seed)
    torch.cuda.synchronize()
    return target, hidden, zq, x, host


def _time_fn(fn, steps, warmup, use_graph):
    """Milliseconds per call of fn(stream): `steps` calls launched back to back
    (or one call captured in a HIP graph and replayed `steps` times) between
    two events."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(warmup, 1)):
            fn(s)
    torch.cuda.synchronize()
    g = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fn(s)
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        g.replay() if g is not None else fn(s)
        start.record(s)
        for _ in range(steps):
            g.replay() if g is not None else fn(s)
        stop.record(s)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    del g
    return ms


def _time_forward(target, hidden, steps, warmup, use_graph=False):
    """Milliseconds per forward over `hidden`, in the kernel family the
    library picks (or SPEC_VERIFY_MATMUL forces)."""
    import torch
    import speculative_decoding_verification_step_amd as sv
    M = hidden.shape[0]
    ws = sv.workspace(target.forward_workspace_bytes(M))
    logits = torch.empty((M, target.vocab), dtype=torch.float32, device="cuda")
    ms = _time_fn(lambda s: target.forward(hidden, logits, ws=ws, stream=s), steps, warmup,
                  use_graph)
    del ws, logits
    return ms


def _time_accept(logits, zq, x, B, K, T, steps, warmup, use_graph=False):
    """Milliseconds per rejection-sampling call alone."""
    import torch
    import speculative_decoding_verification_step_amd as sv
    V = logits.shape[1]
    ws = sv.workspace(sv.accept_workspace_bytes(B, K, V))
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    tl = logits.view(B, K + 1, V)
    ms = _time_fn(lambda s: sv.accept(tl, zq if T > 0 else None, x, T, 0, 0, out_tokens=out,
                                      accept_len=al, ws=ws, stream=s), steps, warmup, use_graph)
    del ws, out, al
    return ms


def _time_step(sv, target, hidden, zq, x, B, K, T, steps, warmup, use_graph, seed=0, stp=0):
    import torch
    M = B * (K + 1)
    V = target.vocab
    ws = sv.workspace(target.workspace_bytes(B, K))
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()

    def one():
        target.step(hidden, zq if T > 0 else None, x, B, K, T, seed, stp, logits, out, al,
                    ws=ws, stream=s)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(warmup, 1)):
            one()
    torch.cuda.synchronize()
    g = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                one()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for _ in range(2):
                g.replay()
        torch.cuda.synchronize()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        start.record(s)
        for i in range(steps):
            if g is not None:
                g.replay()
            else:
                one()
        stop.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    # per-step spread from a second, individually-timed pass (not the headline)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(steps, 50))]
    with torch.cuda.stream(s):
        for a, b in evs:
            a.record(s)
            g.replay() if g is not None else one()
            b.record(s)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    return ms, wall, per, (logits, out, al, ws, s, one)


PROFILE_REPS = 20
PROFILE_BACKLOG_MS = 8.0
PROFILE_MAX_LAUNCHES_PER_STEP = 64


def _profile_backlog_steps(step_ms: float) -> int:
    """Untimed steps queued ahead of each timed one: about
    PROFILE_BACKLOG_MS of GPU work, at least 2."""
    return int(min(200, max(2, math.ceil(PROFILE_BACKLOG_MS / max(step_ms, 1e-3)))))


def _profile_kernels(sv, one, s, step_ms, reps=PROFILE_REPS):
    """Per-kernel times from HIP events that each dispatch records at its own
    start and end, over `reps` steps.  Events on every dispatch slow the step
    by about 5 % on the 768-row workload, so they stay out of the timed loop.
    A launch with events also costs the host more than a short kernel takes
    to run, so each timed step is queued behind a backlog of untimed steps
    (profiling paused; about PROFILE_BACKLOG_MS of GPU work): the GPU reaches
    the timed step busy, at the clock of the timed loop, with the step's
    launches already queued, and runs them back to back as in the timed loop
    instead of waiting on the host.  Returns the per-kernel table and the
    backlog per timed step."""
    import torch
    backlog = _profile_backlog_steps(step_ms)
    sv.profile_begin(reps * PROFILE_MAX_LAUNCHES_PER_STEP)
    try:
        with torch.cuda.stream(s):
            for _ in range(reps):
                sv.profile_pause(True)
                for _ in range(backlog):
                    one()
                sv.profile_pause(False)
                one()
        torch.cuda.synchronize()
    finally:
        kt = sv.profile_end(64)
    return kt, backlog


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _cpu_baseline(host, w, B, K, T, seed):
    """The oracle, as it stands, on a bounded sample of the same workload:
    one request (its K + 1 positions) through the fp64 forward of every block
    and the head (the oracle upcasts each weight matrix from bf16 as it goes,
    so every step reads all the weights, as the GPU step does) and its
    rejection sampling.  Two legs: all the host's BLAS threads, and one
    thread; each reports the median of 5 steps (3 on a 128256-row vocabulary
    with 8 blocks) after one untimed step."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import forward as of, verify as ov
    n_steps = 3 if w.weight_elems() > 1.2e9 else 5
    rows = list(range(K + 1))
    hidden = workload.make_hidden(w, B * (K + 1))[rows]
    g = np.random.default_rng(seed)
    zd = g.standard_normal((1, K, w.vocab)) * math.sqrt(w.d) * w.weight_std
    x = ov.sample_draft_tokens(zd, T, seed, 0)
    es = 2 if w.wdtype == "bf16" else 4
    wbytes = w.weight_elems() * es

    def one(stp):
        z = of.forward(host, hidden)
        ov.verify(z.reshape(1, K + 1, w.vocab), zd, x, T, seed, stp)

    def leg(threads):
        with threadpool_limits(limits=threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            one(0)
            ts = []
            for stp in range(n_steps):
                t0 = time.perf_counter()
                one(stp + 1)
                ts.append(time.perf_counter() - t0)
        med = float(np.median(ts))
        return {"threads": int(used), "median_step_s": med, "steps": n_steps,
                "verified_positions_per_s": len(rows) / med,
                "effective_weight_GBps": wbytes / med / 1e9}

    print(f"[bench] cpu baseline (oracle) on {w.name}: all threads", file=sys.stderr, flush=True)
    all_cores = leg(None)
    print(f"[bench] cpu baseline (oracle) on {w.name}: one thread", file=sys.stderr, flush=True)
    one_core = leg(1)
    return {"value": all_cores["verified_positions_per_s"], "unit": "verified positions/s",
            "cores": all_cores["threads"], "kind": "oracle",
            "sample": f"one request of the {w.name} step ({len(rows)} positions): the oracle's fp64 "
                      f"forward through all {w.n_layers} blocks and the head (weights upcast from "
                      f"storage inside each step) and its rejection sampling; median of {n_steps} "
                      f"steps after one untimed step",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "all_threads": all_cores, "one_thread": one_core}


_CEILINGS: dict = {}


CEILING_WARM_MS = 60.0
CEILING_TIMED_MS = 40.0
CEILING_ROTATE_BYTES = 1.0e9     # beyond the 256 MB last-level cache


def _time_back_to_back(fn, est_ms):
    """Average ms per call of fn(i) over calls queued back to back on one
    stream: about CEILING_WARM_MS of untimed calls first (the GPU reaches the
    timed calls busy, at its loaded clock), then about CEILING_TIMED_MS of
    calls between one pair of events."""
    import torch
    s = torch.cuda.Stream()
    warm = int(min(2000, max(3, math.ceil(CEILING_WARM_MS / est_ms))))
    n = int(min(2000, max(5, math.ceil(CEILING_TIMED_MS / est_ms))))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for i in range(warm):
            fn(i)
        e0.record(s)
        for i in range(n):
            fn(i)
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, n


def _weight_shape(w, label: str):
    """[out, in] of the weight a forward launch streams, by its label."""
    if label.endswith("up_silu"):
        return w.ffn, w.d
    if label.endswith("down_residual"):
        return w.d, w.ffn
    if label.endswith("head"):
        return w.vocab, w.d
    return None


def practical_ceiling(bound: str, w=None, M: int = 0, label: str = ""):
    """A measured practical ceiling beside the published peak, taken once per
    process and shape after the timed work, with the vendor BLAS (hipBLASLt
    through torch) on random bf16 operands, calls queued back to back.
    MFMA-bound: torch.matmul 16384 x 16384 x 8192.  HBM-bound (bf16 weights):
    the dominant launch's own product, F.linear of [M, in] activations with
    its [out, in] weight (no epilogue), the weight rotated over enough copies
    (>= 1 GB) that no call finds it in the last-level cache; rate = (weight +
    activations + output bytes) / time, the same count as the library's own
    weight-streaming roofline."""
    import torch
    import torch.nn.functional as F
    if bound == "mfma":
        key = ("mfma",)
    elif bound == "hbm" and w is not None and w.wdtype == "bf16" and M > 0 \
            and _weight_shape(w, label):
        key = ("hbm", M) + _weight_shape(w, label)
    else:
        return None
    if key in _CEILINGS:
        return _CEILINGS[key]
    gen = torch.Generator(device="cuda").manual_seed(0)
    if bound == "mfma":
        m, n, k = 16384, 16384, 8192
        a = torch.randn((m, k), device="cuda", generator=gen).to(torch.bfloat16)
        b = torch.randn((k, n), device="cuda", generator=gen).to(torch.bfloat16)
        ms, calls = _time_back_to_back(lambda i: torch.matmul(a, b), 3.5)
        res = {"value": 2.0 * m * n * k / (ms / 1e3) / 1e12, "unit": "TFLOP/s",
               "what": f"torch.matmul bf16 16384x16384x8192 (hipBLASLt), random operands, "
                       f"{calls} calls back to back, same run"}
        del a, b
    else:
        n_out, n_in = _weight_shape(w, label)
        wbytes = n_out * n_in * 2
        copies = max(1, math.ceil(CEILING_ROTATE_BYTES / wbytes))
        ws = [(torch.randn((n_out, n_in), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
              for _ in range(copies)]
        x = torch.randn((M, n_in), device="cuda", generator=gen).to(torch.bfloat16)
        nbytes = wbytes + M * n_in * 2 + M * n_out * 2
        ms, calls = _time_back_to_back(lambda i: F.linear(x, ws[i % copies]),
                                       nbytes / (6e12) * 1e3)
        res = {"value": nbytes / (ms / 1e3) / 1e9, "unit": "GB/s",
               "what": f"torch F.linear bf16 [{M},{n_in}] x [{n_out},{n_in}]^T (vendor BLAS), weight "
                       f"rotated over {copies} copies, {calls} calls back to back, same run"}
        del ws, x
    _CEILINGS[key] = res
    torch.cuda.empty_cache()
    return res


def run_point(w, B, K, sigma, T, steps, warmup, use_graph, cpu_baseline, profile=True):
    import torch
    import speculative_decoding_verification_step_amd as sv
    M = B * (K + 1)
    target, hidden, zq, x, host = _device_inputs(w, B, K, T, sigma)
    ms, wall, per, (logits, out, al, ws, s, one) = _time_step(
        sv, target, hidden, zq, x, B, K, T, steps, warmup, use_graph)
    # acceptance statistics (untimed): fresh draft-token draws from q and fresh
    # uniform streams, so the AL law is sampled, not one draw repeated
    als = []
    for stp in range(16):
        xs = _draft_tokens(zq, T, 1000 + stp)
        target.step(hidden, zq if T > 0 else None, xs, B, K, T, 0, stp, logits, out, al, ws=ws)
        als.append(al.cpu().numpy().copy())
    als = np.concatenate(als)
    bytes_, flops = step_work(w, B, K, T)
    # the two halves alone (same launch mode), and the step in the other mode
    sub = max(10, steps // 4)
    fwd_ms = _time_forward(target, hidden, sub, 2, use_graph)
    acc_ms = _time_accept(logits, zq, x, B, K, T, sub, 2, use_graph)
    other_ms, _, other_per, _ = _time_step(sv, target, hidden, zq, x, B, K, T, sub, 2,
                                           not use_graph)
    es = 2 if w.wdtype == "bf16" else 4
    fwd_bytes = w.weight_elems() * es + (w.n_layers + 1) * w.d * 4 + M * w.d * 4 + M * w.vocab * 4
    res = {
        "metric": METRIC,
        "value": M / (ms / 1e3),
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.wdtype == "bf16" else "f32",
        "data": "synthetic (seeded random weights and inputs of the stated shapes)",
        "config": {"workload": w.name, "B": B, "K": K, "M": M, "d": w.d, "ffn": w.ffn,
                   "n_layers": w.n_layers, "vocab": w.vocab, "sigma": sigma, "temperature": T,
                   "launch": "hipgraph" if use_graph else "eager", "parallelism": "none (1 GPU)"},
        "accepted_tokens_per_s": float(als.mean()) * B / (ms / 1e3),
        "mean_accept_len": float(als.mean()),
        "accept_len_hist": np.bincount(als, minlength=K + 2)[1:].tolist(),
        "step_ms_p10_p50_p90": [per[len(per) // 10], per[len(per) // 2], per[(9 * len(per)) // 10]],
        "wall_s_timed": wall,
        "step_bytes": bytes_,
        "step_flops": flops,
        "step_hbm_frac": bytes_ / (ms / 1e3) / (HBM_PEAK_GBS * 1e9),
        "step_mfma_frac": flops / (ms / 1e3) / (MFMA_BF16_PEAK_TFS * 1e12),
        "roofline_step_ms": roofline_time_s(bytes_, flops) * 1e3,
        "forward_ms": fwd_ms,
        "forward_hbm_frac": fwd_bytes / (fwd_ms / 1e3) / (HBM_PEAK_GBS * 1e9),
        "forward_mfma_frac": flops / (fwd_ms / 1e3) / (MFMA_BF16_PEAK_TFS * 1e12),
        "accept_ms": acc_ms,
        ("eager_ms_per_step" if use_graph else "graph_ms_per_step"): other_ms,
        ("eager_step_ms_p10_p50_p90" if use_graph else "graph_step_ms_p10_p50_p90"):
            [other_per[len(other_per) // 10], other_per[len(other_per) // 2],
             other_per[(9 * len(other_per)) // 10]],
    }
    if profile:
        kt, backlog = _profile_kernels(sv, one, s, ms)
        dom = max(kt, key=lambda k: kt[k][1])
        n, tot, b, f = kt[dom]
        avg_s = tot / n / 1e3
        mem_bound = (f / max(b, 1)) < (MFMA_BF16_PEAK_TFS / HBM_PEAK_GBS * 1e3)
        if mem_bound or w.wdtype != "bf16":
            roof = {"bound": "hbm", "achieved": b / n / avg_s / 1e9, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s"}
        else:
            roof = {"bound": "mfma", "achieved": f / n / avg_s / 1e12, "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        ceil = practical_ceiling(roof["bound"], w, M, dom)
        if ceil:
            roof["ceiling"] = dict(ceil, frac=roof["achieved"] / ceil["value"])
        roof["traffic"] = measured_traffic(w.name, dom) if (B, K) == (w.B, w.K) else None
        roof["kernel"] = dom
        roof["avg_launch_us"] = avg_s * 1e6
        roof["algorithmic_bytes_per_launch"] = b / n
        roof["algorithmic_flops_per_launch"] = f / n
        res["roofline"] = roof
        res["kernels"] = {k: {"launches": v[0] // PROFILE_REPS, "ms_per_step": v[1] / PROFILE_REPS,
                              "gbs": v[2] / max(v[1], 1e-9) / 1e6} for k, v in kt.items()}
        res["kernels_profile_steps"] = PROFILE_REPS
        res["kernels_profile_backlog_steps"] = backlog
        res["kernels_ms_per_step_sum"] = sum(v[1] for v in kt.values()) / PROFILE_REPS
    if cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline(host, w, B, K, T, 0)
    del target, hidden, zq, x, logits, out, al, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


K_TABLE_B = (1, 4, 16, 64)
K_TABLE_K = tuple(range(9))
K_TABLE_CHOOSE_B = (1, 2, 4, 8, 16, 32, 64)
K_TABLE_DRAFT_C = (0.0, 0.05)


def _k_table(a):
    """Hardware-aware draft length: the verification step is timed on this GPU
    at every B x K of the sweep grid (rows M = B (K + 1)), AL(K) is measured
    on the same synthetic drafts, and the library picks the K of highest
    goodput AL / (T_verif + T_draft) per batch size, for a free draft and for
    a draft costing c * T_verif(B) per token."""
    import torch
    import speculative_decoding_verification_step_amd as sv
    w = workload.WORKLOADS["8b-shaped-sweep"]
    for sigma in workload.SWEEP_SIGMA:
        times: dict = {}
        al = [1.0]
        for K in K_TABLE_K:
            for B in K_TABLE_B:
                target, hidden, zq, x, _ = _device_inputs(w, B, K, 1.0, sigma)
                ms, _, _, (logits, out, alb, ws, _, _) = _time_step(
                    sv, target, hidden, zq, x, B, K, 1.0, 20, 2, a.graph)
                times.setdefault(B * (K + 1), []).append(ms)
                if B == K_TABLE_B[-1] and K > 0:
                    als = []
                    for stp in range(16):
                        xs = _draft_tokens(zq, 1.0, 2000 + stp)
                        target.step(hidden, zq, xs, B, K, 1.0, 0, stp, logits, out, alb, ws=ws)
                        als.append(alb.cpu().numpy().copy())
                    al.append(float(np.concatenate(als).mean()))
                del hidden, zq, x, logits, out, alb, ws
                torch.cuda.synchronize()
        m_rows = sorted(times)
        t_verif = [float(np.mean(times[m])) for m in m_rows]
        res = {"k_table": w.name, "sigma": sigma, "temperature": 1.0,
               "launch": "hipgraph" if a.graph else "eager",
               "al_measured": al, "rows": m_rows, "t_verif_ms": t_verif, "choice": {}}
        for c in K_TABLE_DRAFT_C:
            t_b = {B: float(np.interp(B, m_rows, t_verif)) for B in K_TABLE_CHOOSE_B}
            draft = [[c * K * t_b[B] for K in K_TABLE_K] for B in K_TABLE_CHOOSE_B]
            k, g = sv.choose_k(m_rows, t_verif, al, list(K_TABLE_CHOOSE_B), draft)
            res["choice"][f"c={c}"] = {
                str(B): {"K": int(k[i]), "goodput_tokens_per_ms_per_request": float(g[i]),
                         "speedup_vs_K0": float(g[i] * t_b[B])}
                for i, B in enumerate(K_TABLE_CHOOSE_B)}
        print(json.dumps(res), flush=True)


MOE_B = (1, 2, 4, 8, 16, 32, 64)
MOE_K = tuple(range(9))


def _moe_bench(a):
    """Verification step of the 64-expert top-6 MoE stack over B x K: the
    forward (reporting the distinct experts each block touched, so the bytes
    streamed are the experts actually used) plus rejection sampling; then the
    library's goodput-optimal K per batch size from the measured times and
    acceptance lengths (Cohere DSD: for MoE the optimum need not fall with B)."""
    import torch
    import speculative_decoding_verification_step_amd as sv
    w = workload.MOE_WORKLOADS["moe-64e-top6-b1-k4"]
    T = 1.0
    for sigma in workload.SWEEP_SIGMA:
        model = workload.make_moe_model(w, sigma=sigma)

        def dev(x):
            return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        L, E, d, f, V = w.n_layers, w.n_experts, w.d, w.ffn, w.vocab
        pr, pu, pd = sv.pack(dev(model["w_router"])), sv.pack(dev(model["w_up"]).reshape(L * E, f, d)), \
            sv.pack(dev(model["w_down"]).reshape(L * E, d, f))
        gain = torch.from_numpy(model["gain"]).cuda()
        target = sv.MoEModel(pr, pu, pd, gain, sv.pack(dev(model["w_head"])), (L, E, d, f, V), w.top_k)
        drafter = sv.MoEModel(pr, pu, pd, gain, sv.pack(dev(model["w_draft_head"])), (L, E, d, f, V),
                              w.top_k)
        del model
        times, al_by_k, points = {}, {0: 1.0}, []
        expert_bytes = 2.0 * d * f * 2
        for K in MOE_K:
            for B in MOE_B:
                M = B * (K + 1)
                g = np.random.default_rng(1000 * B + K)
                hidden = torch.from_numpy(g.standard_normal((M, d)).astype(np.float32)).cuda()
                zq = drafter.forward(hidden).view(B, K + 1, V)[:, :K].contiguous()
                x = _draft_tokens(zq, T, 7)
                logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
                active = torch.zeros(L, dtype=torch.int32, device="cuda")
                fws = sv.workspace(target.workspace_bytes(M))
                aws = sv.workspace(sv.accept_workspace_bytes(B, K, V))
                out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
                al = torch.empty((B,), dtype=torch.int32, device="cuda")

                def step(s, stp=0):
                    target.forward(hidden, logits, active=active, ws=fws, stream=s)
                    sv.accept(logits.view(B, K + 1, V), zq if K else None, x if K else None, T, 0, stp,
                              out_tokens=out, accept_len=al, ws=aws, stream=s)
                ms = _time_fn(step, 20, 2, a.graph)
                act = cpu_ints(active)
                if K and B == MOE_B[-1]:
                    als = []
                    for stp in range(16):
                        xs = _draft_tokens(zq, T, 3000 + stp)
                        target.forward(hidden, logits, active=active, ws=fws)
                        sv.accept(logits.view(B, K + 1, V), zq, xs, T, 0, stp, out_tokens=out,
                                  accept_len=al, ws=aws)
                        als.append(al.cpu().numpy().copy())
                    al_by_k[K] = float(np.concatenate(als).mean())
                bytes_ = sum(act) * expert_bytes + L * E * d * 2 + V * d * 2 + M * d * 4 + \
                    2 * M * V * 4 + (B * K * V * 4 if K else 0)
                times.setdefault(M, []).append(ms)
                rec = {"moe": w.name, "sigma": sigma, "B": B, "K": K, "M": M, "ms_per_step": ms,
                       "active_experts_per_block": act,
                       # distinct experts if every position picked top_k of E uniformly
                       "expected_active_uniform": E * (1.0 - (1.0 - w.top_k / E) ** M),
                       "step_bytes": bytes_, "step_hbm_frac": bytes_ / (ms / 1e3) / (HBM_PEAK_GBS * 1e9),
                       "verified_positions_per_s": M / (ms / 1e3),
                       "launch": "hipgraph" if a.graph else "eager"}
                points.append(rec)
                print(json.dumps(rec), flush=True)
                del hidden, zq, x, logits, fws, aws
        m_rows = sorted(times)
        t_verif = [float(np.mean(times[m])) for m in m_rows]
        al = [al_by_k[k] for k in MOE_K]
        res = {"moe_k_table": w.name, "sigma": sigma, "al_measured": al, "rows": m_rows,
               "t_verif_ms": t_verif, "choice": {}}
        for c in K_TABLE_DRAFT_C:
            t_b = {B: float(np.interp(B, m_rows, t_verif)) for B in MOE_B}
            draft = [[c * K * t_b[B] for K in MOE_K] for B in MOE_B]
            k, gp = sv.choose_k(m_rows, t_verif, al, list(MOE_B), draft)
            res["choice"][f"c={c}"] = {str(B): {"K": int(k[i]), "speedup_vs_K0": float(gp[i] * t_b[B])}
                                       for i, B in enumerate(MOE_B)}
        print(json.dumps(res), flush=True)
        del target, drafter, pr, pu, pd
        torch.cuda.empty_cache()


def cpu_ints(t):
    return [int(v) for v in t.cpu().tolist()]


ATTN_K = (0, 1, 3, 7, 15)


def _attention_bench(a):
    """Paged attention of the T = K + 1 verified positions over a full KV
    cache: time per call (eager, back to back), the KV bytes it must read
    once, and the fraction of HBM bandwidth; the attention GEMM-M per KV head
    is G (K + 1) (NVIDIA co-design post, 'Draft length and attention
    performance').  Cache contents are seeded random bf16 drawn on the GPU."""
    import torch
    import speculative_decoding_verification_step_amd as sv
    for name, c in workload.ATTN_WORKLOADS.items():
        B, Hq, Hkv, Dh, ctx = c["B"], c["Hq"], c["Hkv"], c["Dh"], c["ctx"]
        G = Hq // Hkv
        for K in ATTN_K:
            T = K + 1
            mb = -(-(ctx + T) // workload.KV_BLOCK)
            nb = B * mb
            gen = torch.Generator(device="cuda").manual_seed(1234)
            kc = torch.randn((nb, Hkv, workload.KV_BLOCK, Dh), generator=gen, device="cuda").to(torch.bfloat16)
            vc = torch.randn((nb, Hkv, Dh, workload.KV_BLOCK), generator=gen, device="cuda").to(torch.bfloat16)
            perm = torch.randperm(nb, generator=gen, device="cuda").to(torch.int32)
            table = perm.view(B, mb).contiguous()
            ctx_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
            q = torch.randn((B, T, Hq, Dh), generator=gen, device="cuda").to(torch.bfloat16)
            kn = torch.randn((B, T, Hkv, Dh), generator=gen, device="cuda").to(torch.bfloat16)
            vn = torch.randn((B, T, Hkv, Dh), generator=gen, device="cuda").to(torch.bfloat16)
            out = torch.empty((B, T, Hq, Dh), dtype=torch.float32, device="cuda")
            n = sv.attention_workspace_bytes(B, T, Hq, Hkv, Dh, mb)
            ws = sv.workspace(n) if n else None
            sv.kv_append(kn, vn, kc, vc, table, ctx_len)
            scale = 1.0 / math.sqrt(Dh)
            ms = _time_fn(lambda s: sv.attention(q, kc, vc, table, ctx_len, scale, out=out, ws=ws,
                                                 stream=s), 50, 5, a.graph)
            def one_call():
                sv.attention(q, kc, vc, table, ctx_len, scale, out=out, ws=ws)
                sv.kv_append(kn, vn, kc, vc, table, ctx_len)

            kt, _ = _profile_kernels(sv, one_call, torch.cuda.Stream(), ms)
            kv_bytes = B * Hkv * (ctx + T) * Dh * 2 * 2
            io_bytes = B * T * Hq * Dh * (2 + 4)
            flops = 4.0 * B * Hq * T * (ctx + (T + 1) / 2.0) * Dh
            main = kt.get("attention", (PROFILE_REPS, PROFILE_REPS * ms, 0, 0))
            comb = kt.get("attention_combine", (0, 0.0, 0, 0))
            app = kt.get("kv_append", (PROFILE_REPS, 0.0, 0, 0))
            comb_us = comb[1] / comb[0] * 1e3 if comb[0] else 0.0
            attn_us = main[1] / main[0] * 1e3 + comb_us    # both launches of one call
            res = {"attention": name, "B": B, "Hq": Hq, "Hkv": Hkv, "G": G, "Dh": Dh, "ctx": ctx,
                   "K": K, "T": T, "gemm_m_per_kv_head": G * T,
                   "launch": "hipgraph" if a.graph else "eager",
                   "us_per_call": ms * 1e3,
                   "kernel_us": attn_us,
                   "combine_us": comb_us,
                   "append_us": app[1] / app[0] * 1e3 if app[0] else 0.0,
                   "kv_bytes": kv_bytes,
                   "achieved_GBps": (kv_bytes + io_bytes) / (attn_us * 1e-6) / 1e9,
                   "hbm_frac": (kv_bytes + io_bytes) / (attn_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                   "TFLOPs": flops / (attn_us * 1e-6) / 1e12,
                   "verified_positions_per_s": B * T / (ms / 1e3)}
            print(json.dumps(res), flush=True)
            del kc, vc, q, kn, vn, out, ws, table, perm, ctx_len
            torch.cuda.empty_cache()


CYCLE_B = (1, 4, 16, 64)
CYCLE_K = tuple(range(7))      # K = 0: plain decoding
CYCLE_EXITS = (0, 1)           # drafter = the target's first n blocks, final norm and head
CYCLE_STATS = 32               # cycles per point for the acceptance statistics


def _cycle_bench(a):
    """Whole speculative cycles on the 8B-shaped target (publishertech
    section 2, "Theoretical Speedup Equation"): the drafter is an early exit
    of the target (its first n blocks, its final norm and head; no weights of
    its own), tokens feed back through an embedding table, and one cycle is
    the draft loop, the verification of the K + 1 positions and the next
    input token, all on the device.  Per drafter, B and K: ms per cycle
    (eager, and one captured graph replayed), emitted tokens per second,
    the measured acceptance rate alpha and draft cost c (one draft step over
    one plain decoding step), and the speedup over plain decoding (K = 0)
    beside the pages' model E[N] / (1 + K c) with E[N] = (1 - alpha^(K+1)) /
    (1 - alpha)."""
    import torch
    import speculative_decoding_verification_step_amd as sv
    w = workload.WORKLOADS["8b-shaped-b1-k4"]
    T = 1.0 if a.T is None else a.T
    target, _, _ = _device_models(w, w.sigma)
    up, down, gain, head = target._keep
    table = torch.from_numpy(workload.make_embedding(w)).cuda()
    d, ffn, V = w.d, w.ffn, w.vocab
    for n_exit in CYCLE_EXITS:
        g_d = torch.cat([gain[:n_exit], gain[-1:]]).contiguous()
        drafter = sv.Model(up, down, g_d, head, layout="tiled", dims=(n_exit, d, ffn, V))
        for B in CYCLE_B:
            start = torch.from_numpy(workload.make_start_tokens(V, B, seed=B)).cuda()
            cur = start.clone()
            dws = sv.workspace(drafter.draft_workspace_bytes(B))
            dtok = torch.empty((B, 1), dtype=torch.int32, device="cuda")
            dlog = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
            t_draft = _time_fn(lambda s: drafter.draft(table, cur, 1, T, 1, 0, dtok, dlog, dws, s),
                               20, 2, False)
            rows = []
            for K in CYCLE_K:
                dr = drafter if K else None
                ws = sv.workspace(sv.cycle_workspace_bytes(target, dr, B, K))
                out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
                al = torch.empty((B,), dtype=torch.int32, device="cuda")
                cur = start.clone()
                als = []
                for stp in range(CYCLE_STATS):
                    sv.cycle(target, dr, table, cur, K, T, 7, stp, out, al, ws)
                    als.append(al.clone())
                al_all = torch.stack(als).cpu().numpy()
                cur = start.clone()

                def one(s):
                    sv.cycle(target, dr, table, cur, K, T, 7, 0, out, al, ws, stream=s)
                ms = _time_fn(one, 20, 2, False)
                ms_graph = _time_fn(one, 20, 2, True)
                mean_al = float(al_all.mean())
                alpha = float((al_all - 1).sum() / np.minimum(al_all, K).sum()) if K else None
                rows.append({"K": K, "ms_per_cycle": ms, "graph_ms_per_cycle": ms_graph,
                             "mean_accept_len": mean_al, "alpha": alpha,
                             "tokens_per_s": B * mean_al / (ms / 1e3)})
                del ws, out, al
            t0 = rows[0]["ms_per_cycle"]
            c = t_draft / t0
            for r in rows:
                K, alpha = r["K"], r["alpha"]
                en = 1.0 if K == 0 else ((1 - alpha ** (K + 1)) / (1 - alpha) if alpha < 1 else K + 1.0)
                rec = {"cycle": w.name, "drafter": f"exit-{n_exit}", "B": B, "T": T, **r,
                       "draft_step_ms": t_draft, "c": c,
                       "speedup_measured": r["tokens_per_s"] / rows[0]["tokens_per_s"],
                       "speedup_model": en / (1 + K * c),
                       "launch": "eager (graph replay beside it)"}
                print(json.dumps(rec), flush=True)
            best = max(rows, key=lambda r: r["tokens_per_s"])
            print(json.dumps({"cycle_best": w.name, "drafter": f"exit-{n_exit}", "B": B, "K": best["K"],
                              "speedup": best["tokens_per_s"] / rows[0]["tokens_per_s"], "c": c}),
                  flush=True)
            del dws, dtok, dlog
        del drafter
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(workload.WORKLOADS))
    ap.add_argument("--B", type=int)
    ap.add_argument("--K", type=int)
    ap.add_argument("--sigma", type=float)
    ap.add_argument("--T", type=float)
    ap.add_argument("--graph", action="store_true",
                    help="time HIP graph replays as the headline (default: eager launches; the "
                         "other mode is reported beside it)")
    ap.add_argument("--eager", action="store_true", help=argparse.SUPPRESS)  # the default
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--no-nested", action="store_true",
                    help="headline workload only (no nested records of the other workloads)")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--moe", action="store_true",
                    help="mixture-of-experts target: step time, experts touched and HBM roofline per "
                         "B x K, and the goodput-optimal draft length per batch size")
    ap.add_argument("--attention", action="store_true",
                    help="paged attention of the verified positions: time and HBM roofline per "
                         "workload and draft length")
    ap.add_argument("--k-table", action="store_true",
                    help="measure T_verif(M) and AL(K) on the sweep stack and print the "
                         "goodput-optimal draft length per batch size")
    ap.add_argument("--crossover", action="store_true",
                    help="forward-only times of both MFMA kernel families over B*(K+1)")
    ap.add_argument("--cycle", action="store_true",
                    help="whole speculative cycles (draft loop + verification) with early-exit "
                         "drafters: tokens/s, acceptance, draft cost and speedup over plain decoding")
    ap.add_argument("--calib-copy", action="store_true",
                    help="finish with one plain 256 MiB device copy (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              "(requests are independent: several GPUs would each verify their own share of "
              "the batch, and this program measures one)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if a.sweep:
        w = workload.WORKLOADS["8b-shaped-sweep"]
        for sigma in workload.SWEEP_SIGMA:
            for B in workload.SWEEP_B:
                for K in workload.SWEEP_K:
                    r = run_point(w, B, K, sigma, 1.0, max(20, a.steps // 4), 3, a.graph,
                                  False, profile=False)
                    print(json.dumps(r), flush=True)
        return
    if a.k_table:
        _k_table(a)
        return
    if a.attention:
        _attention_bench(a)
        return
    if a.moe:
        _moe_bench(a)
        return
    if a.cycle:
        _cycle_bench(a)
        return
    if a.crossover:
        # forward-only time per row count with each MFMA family forced: the
        # HBM-bound streaming kernel against the LDS-staged GEMM
        import torch
        w = workload.WORKLOADS["8b-shaped-sweep"]
        target, _, _ = _device_models(w, w.sigma)
        bytes_w = w.weight_elems() * 2
        for M in CROSSOVER_ROWS:
            hidden = torch.from_numpy(workload.make_hidden(w, M)).cuda()
            row = {"crossover": w.name, "M": M}
            for kind in ("skinny", "tiled"):
                os.environ["SPEC_VERIFY_MATMUL"] = kind
                ms = _time_forward(target, hidden, 20, 2)
                row[kind] = {"ms": ms, "weight_TBps": bytes_w / (ms / 1e3) / 1e12,
                             "TFLOPs": 2.0 * M * w.weight_elems() / (ms / 1e3) / 1e12}
            os.environ.pop("SPEC_VERIFY_MATMUL", None)
            row["auto_ms"] = _time_forward(target, hidden, 20, 2)
            row["faster"] = min(("skinny", "tiled"), key=lambda k: row[k]["ms"])
            print(json.dumps(row), flush=True)
        return

    w = workload.WORKLOADS[a.workload]
    B = a.B or w.B
    K = w.K if a.K is None else a.K
    sigma = w.sigma if a.sigma is None else a.sigma
    T = w.temperature if a.T is None else a.T
    print(f"[bench] {w.name}: B={B} K={K}, {a.steps} timed steps", file=sys.stderr, flush=True)
    res = run_point(w, B, K, sigma, T, a.steps, a.warmup, a.graph, not a.no_cpu_baseline,
                    profile=not a.no_profile)
    if w.name == HEADLINE and (a.B, a.K, a.sigma, a.T) == (None, None, None, None) and not a.no_nested:
        res["workloads"] = {}
        for name in NESTED:
            wn = workload.WORKLOADS[name]
            print(f"[bench] nested {name}: B={wn.B} K={wn.K}", file=sys.stderr, flush=True)
            r = run_point(wn, wn.B, wn.K, wn.sigma, wn.temperature, a.steps, a.warmup, a.graph,
                          False, profile=not a.no_profile)
            res["workloads"][name] = {k: r[k] for k in NESTED_KEYS if k in r}
            res["workloads"][name]["verified_positions_per_s"] = r["value"]
    print(json.dumps(res), flush=True)
    if a.calib_copy:
        # a plain copy of known size: 256 MiB read + 256 MiB written, so the
        # HBM byte counters of the kernels above can be scaled by it
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)        # one elementwise kernel: read + write 256 MiB
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
