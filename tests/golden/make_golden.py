"""Writes c1_oracle_summary.json from the oracle alone (drift check)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import tp_inputs  # noqa: E402


def summary():
    w = tp_inputs.C1
    inp = tp_inputs.make_inputs(w, seed=0)
    ranks = [O.rank_forward(inp["x"], inp.values, w.tp_degree, r, 0, 0, bf16=False)
             for r in range(w.tp_degree)]
    y = O.partial_reduce([r["p_mlp"] for r in ranks], O.rowwise_bias(inp.values))
    rng = np.random.default_rng(123)
    idx = [(int(a), int(b)) for a, b in zip(rng.integers(0, y.shape[0], 16),
                                             rng.integers(0, y.shape[1], 16))]
    return {
        "workload": w.name,
        "seed": 0,
        "shape": list(y.shape),
        "sum": float(y.sum()),
        "sum_sq": float((y * y).sum()),
        "max_abs": float(np.abs(y).max()),
        "samples": [[i, j, float(y[i, j])] for i, j in idx],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "c1_oracle_summary.json"), "w") as f:
        json.dump(summary(), f, indent=1)
        f.write("\n")
