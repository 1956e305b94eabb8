#!/usr/bin/env python3
"""Writes tests/golden/bf16_stack_spread.json.

For every full-size bf16 workload, the oracle's logits on the rows the GPU
forward tests sample are computed twice: with fp64 accumulation (the
reference) and with fp32 accumulation in the same block order and the same
bf16 rounding points.  Both are valid evaluations of "bf16 inputs, fp32 or
better accumulation"; their distance is the spread that accumulation order
alone produces through the stack, and it bounds how closely any fp32
implementation (the GPU's included) can be expected to match the reference
on a full stack.  Calls only ``workload`` and ``oracle``.

    python tests/golden/make_stack_spread.py
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

ROWS = {
    "8b-shaped-b1-k4": [0, 1, 2, 3, 4],
    "70b-layer-share-b8-k4": [0, 4, 17, 35, 39],
    "large-batch-b256-k2": [0, 1, 2, 383, 765, 767],
}


def main():
    out = {"note": __doc__.strip().splitlines()[2:9], "workloads": {}}
    for name, rows in ROWS.items():
        t0 = time.time()
        w = workload.WORKLOADS[name]
        model = workload.make_model(w, draft_head=False)
        hidden = workload.make_hidden(w)[rows]
        z64 = of.forward(model, hidden)
        z32 = of.forward(model, hidden, accum="f32")
        d = np.abs(z32 - z64)
        out["workloads"][name] = {"rows": rows, "max_abs": float(d.max()),
                                  "mean_abs": float(d.mean()),
                                  "p999_abs": float(np.quantile(d, 0.999))}
        print(name, out["workloads"][name], f"{time.time() - t0:.0f}s", flush=True)
        del model
    with open(os.path.join(HERE, "bf16_stack_spread.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
