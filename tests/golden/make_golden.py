"""Writes oracle_small.json: a regression fixture produced by the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
It imports only the oracle and the test-side problem generator (no GPU code).
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from pins import rand_problem  # noqa: E402

SEED, SHAPE = 77, [1, 24, 2, 3, 4, 1]
p = rand_problem(SEED, *SHAPE)
out = oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"])
gold = {
    "what": "oracle y and final state on a seeded small problem (regression guard only; "
            "the oracle's correctness is pinned by tests/pins.py, not by this file)",
    "seed": SEED, "shape": SHAPE,
    "y_head": [float(v) for v in out["y"].ravel()[:24]],
    "final_head": [float(v) for v in out["final"].ravel()[:24]],
    "y_sum": float(np.sum(out["y"])),
}
with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
    json.dump(gold, f, indent=1)
print("wrote", os.path.join(HERE, "oracle_small.json"))
