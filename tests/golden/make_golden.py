"""Write tests/golden/config1_oracle.json from the CPU oracle alone.

The pages print no worked example for the recurrence, so the only stored
expected values are the oracle's own, for the small fp32 workload
(L=32, B=4, d=64, one direction, alpha=1, seed 1).  They freeze the oracle and
the input generator against silent drift; the oracle itself is pinned by
tests/test_oracle_pins.py.  Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from parallelizable_recurrent_units_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

SAMPLES = [(0, 0, 0), (5, 1, 17), (31, 3, 63), (16, 2, 40)]   # (t, b, j)


def compute():
    w = WORKLOADS[1]
    inp = make_inputs(w, seed=1)
    U = oracle.layer_U(inp["x"], inp["W"], False, w.L, w.B, w.ndir, w.d)
    out = oracle.forward(U, inp["x"], inp["v"], inp["b"], inp["c0"], w.alpha)
    rec = {
        "workload": w.name,
        "seed": 1,
        "inputs_sha256": {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
                          for k, v in sorted(inp.items())},
        "samples": [],
        "h_sum": float(out["h"].sum()),
        "c_last_sum": float(out["c_last"].sum()),
    }
    for t, b, j in SAMPLES:
        rec["samples"].append({"t": t, "b": b, "j": j,
                               "U_f": float(U[t, b, 0, 0, j]),
                               "h": float(out["h"][t, b, 0, j]),
                               "c": float(out["c"][t, b, 0, j])})
    return rec


if __name__ == "__main__":
    with open(os.path.join(HERE, "config1_oracle.json"), "w") as f:
        json.dump(compute(), f, indent=1)
        f.write("\n")
