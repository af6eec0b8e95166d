"""Writes tests/golden/c1_rank0.json from the oracle alone (run from the repository root).

Workload: 2 heads, d = 64, a 256-token sequence in 4 chunks of 64, rank 0, non-causal, fp32
inputs from the seeded generator (workload key 1). Stored: every LSE value and three output rows
per head. The test recomputes them with the oracle, so a later change to the oracle's arithmetic
shows up as a difference here.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from long_context_sequence_amd import configs, inputs  # noqa: E402

ROWS = [0, 31, 63]


def compute():
    wl = configs.C1
    q = inputs.widen(inputs.workload_tensor(wl, "q", 0))
    k = inputs.widen(inputs.workload_kv(wl, "k"))
    v = inputs.widen(inputs.workload_kv(wl, "v"))
    o, lse = oracle.rank_forward(q, k, v, 0, wl.causal)
    return {"workload": wl.name, "rank": 0, "rows": ROWS,
            "lse": lse.tolist(), "o_rows": o[:, ROWS].tolist()}


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_rank0.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=0)
    print("wrote", out)
