"""Writes tests/golden/tiny_gru.json from the oracle alone (sequential states and the
Newton iteration counts / residual histories of the 4-channel, 64-step GRU workload).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from nonlinear_rnn_evaluation_amd import workloads as WL  # noqa: E402


def main():
    w = WL.get_workload("tiny_gru")
    p = {k: WL.as_f64(v) for k, v in WL.generate(w).items()}
    seq = O.sequential(w.cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"])
    out = {"workload": w.describe(), "sequential": seq.reshape(-1).tolist()}
    for name, mode in (("full", O.JAC_FULL), ("diag", O.JAC_DIAG)):
        r = O.newton_dense(w.cell, p["W"], p["U"], p["b_x"], p["b_h"], p["x"], p["h0"],
                           w.max_iters, w.tol, mode)
        out[name] = {"iters": r["iters"], "status": r["status"], "rhos": r["rhos"]}
    with open(os.path.join(ROOT, "tests", "golden", "tiny_gru.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
