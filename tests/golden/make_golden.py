"""Writes brute_small.json: tiny attention cases evaluated by the 40-digit
decimal brute force in ``oracle/brute.py`` (and nothing else).

The pages print no worked example, so this fixture is a regression pin of the
float64 oracle against the independent decimal computation.  Re-run with
``python tests/golden/make_golden.py`` from the repository root.
"""
import json
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle.brute import brute_fwd_decimal  # noqa: E402


def main():
    rng = np.random.default_rng(4242)
    cases = []
    for n, d, causal in ((3, 2, False), (4, 3, True), (7, 4, False), (9, 2, True)):
        q = np.round(rng.standard_normal((n, d)) * 1.5, 6)
        k = np.round(rng.standard_normal((n, d)) * 1.5, 6)
        v = np.round(rng.standard_normal((n, d)), 6)
        scale = 1.0 / math.sqrt(d)
        o, lse = brute_fwd_decimal(q, k, v, scale, causal)
        cases.append({
            "n": n, "d": d, "causal": causal, "scale": scale,
            "q": q.tolist(), "k": k.tolist(), "v": v.tolist(),
            "o": [[float(x) for x in r] for r in o],
            "lse": [float(x) for x in lse],
        })
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "brute_small.json")
    with open(out, "w") as f:
        json.dump({"source": "oracle/brute.py brute_fwd_decimal, 40 significant digits",
                   "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
