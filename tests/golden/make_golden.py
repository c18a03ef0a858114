"""Writes the stored expected values under tests/golden/.

Calls only the fp64 oracle (oracle/).  Run from the repository root:
    python tests/golden/make_golden.py

scalar_T2.json -- the hand-checkable case the Darknet LSTM walkthrough
recommends for bookkeeping (hidden, input and batch size 1, two steps,
simple weights), once with a zero and once with a non-zero initial state, so
that the initial-state path is separated from leakage between sequences.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import oracle  # noqa: E402

# W is [4H, H+I] = [4, 2]: rows i, f, g, o; columns [w_h, w_x]
CASE = dict(
    W=[[0.5, -0.3], [0.2, 0.4], [-0.6, 0.1], [0.3, 0.7]],
    b=[0.1, -0.2, 0.05, 0.0],
    x=[[[0.8]], [[-0.5]]],
    dy=[[[0.7]], [[-1.1]]],
    dhT=[[0.25]],
    dcT=[[-0.5]],
)
STATES = {"zero_state": ([[0.0]], [[0.0]]), "nonzero_state": ([[0.3]], [[-0.4]])}


def main():
    out = {"source": "tests/golden/make_golden.py (fp64 oracle)", "inputs": CASE, "cases": {}}
    for name, (h0, c0) in STATES.items():
        inp = {k: np.array(v, dtype=np.float64) for k, v in CASE.items()}
        inp["h0"], inp["c0"] = np.array(h0), np.array(c0)
        fw = oracle.fwd(inp["x"], inp["W"], inp["b"], inp["h0"], inp["c0"])
        bw = oracle.bwd(inp["x"], inp["W"], inp["h0"], inp["c0"], fw, inp["dy"], inp["dhT"], inp["dcT"])
        rec = {"h0": h0, "c0": c0}
        for k in ("y", "hT", "cT", "gates", "cell"):
            rec[k] = fw[k].tolist()
        for k in ("dx", "dW", "db", "dh0", "dc0"):
            rec[k] = bw[k].tolist()
        out["cases"][name] = rec
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "scalar_T2.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
