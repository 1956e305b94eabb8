#!/usr/bin/env python3
"""Writes tests/golden/bf16_stack_spread.json.

For every full-size bf16 workload, the oracle's logits on every row of the
step (all B*(K+1) positions, the rows the GPU step test compares) are
computed with fp64 accumulation (the reference) and in fp32 (matmuls,
residual stream, norm and SiLU in fp32, the same bf16 rounding points) in
four summation orders of the reduction index.  Every one is a valid
evaluation of "bf16 inputs, fp32 accumulation"; their distance from the
reference is the spread that rounding alone produces through the stack.  The
maximum over a few rows is set by the single worst cascade of bf16 rounding
flips, so it varies between orders; the envelope over the orders (largest
max and p99.9, mean of the means) is what the GPU is held to.  Calls only
``workload`` and ``oracle``.  The 8B-shaped sweep (B x K over the same
stack) takes the first 576 rows, the largest B*(K+1) of the sweep; every
point of the sweep steps over a prefix of them.

    python tests/golden/make_stack_spread.py [name ...]   (default: all; the
    named workloads are recomputed and merged into the existing file)
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workload  # noqa: E402
from oracle import forward as of  # noqa: E402

ORDERS = (0, 1, 2, 3)
# workload -> rows of the step (None: its own B * (K + 1))
NAMES = {"8b-shaped-b1-k4": None, "70b-layer-share-b8-k4": None, "large-batch-b256-k2": None,
         "8b-shaped-sweep": max(workload.SWEEP_B) * (max(workload.SWEEP_K) + 1)}
PATH = os.path.join(HERE, "bf16_stack_spread.json")


def main(names):
    out = {"note": __doc__.strip().splitlines()[2:14], "workloads": {}}
    if os.path.exists(PATH) and set(names) != set(NAMES):
        with open(PATH) as f:
            out["workloads"] = json.load(f)["workloads"]
    for name in names:
        t0 = time.time()
        w = workload.WORKLOADS[name]
        model = workload.make_model(w, draft_head=False)
        hidden = workload.make_hidden(w, NAMES[name])
        z64 = of.forward(model, hidden)
        per = []
        for order in ORDERS:
            d = np.abs(of.forward(model, hidden, accum="f32", k_order=order) - z64)
            per.append({"k_order": order, "max_abs": float(d.max()), "mean_abs": float(d.mean()),
                        "p999_abs": float(np.quantile(d, 0.999))})
            print(name, per[-1], flush=True)
            del d
        out["workloads"][name] = {"rows": "all", "n_rows": int(hidden.shape[0]),
                                  "max_abs": max(r["max_abs"] for r in per),
                                  "mean_abs": float(np.mean([r["mean_abs"] for r in per])),
                                  "p999_abs": max(r["p999_abs"] for r in per),
                                  "orders": per}
        print(name, out["workloads"][name], f"{time.time() - t0:.0f}s", flush=True)
        del model
    with open(PATH, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main(sys.argv[1:] or list(NAMES))
