"""Write oracle_small.json: the CPU oracle's outputs on one small seeded case.

Imports only the oracle and the seeded input generator.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from moe_inputs import Workload, make_inputs  # noqa: E402

CASE = dict(name="golden", T=12, d=8, E=5, k=2, F=6, dtype="fp32", w_std=0.5,
            seed=77)


def compute():
    inp = make_inputs(Workload(**CASE))
    k = CASE["k"]
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, k)
    bwd = O.layer_backward(fwd, inp.dy, inp.x, inp.wr, inp.w1, inp.w2, k)
    out = {"case": CASE}
    for key in ("idx", "counts", "offsets", "dest", "src"):
        out[key] = np.asarray(fwd[key]).reshape(-1).tolist()
    for key in ("w", "y"):
        out[key] = np.asarray(fwd[key]).reshape(-1).tolist()
    for key in ("dx", "dwr"):
        out[key] = np.asarray(bwd[key]).reshape(-1).tolist()
    out["dw1_sum"] = float(np.sum(bwd["dw1"]))
    out["dw2_sum"] = float(np.sum(bwd["dw2"]))
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(compute(), f, indent=1)
        f.write("\n")
