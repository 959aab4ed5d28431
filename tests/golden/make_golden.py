"""Writes tests/golden/tiny_causal.json from the fp64 oracle (and nothing else).

The pages print no attention values, so this fixture is a regression pin of the oracle on a
tiny causal case (N = 6, d = 4): it catches accidental changes to the oracle's arithmetic.
The case follows the shape rules of "Systems and Parallelism" (CS336 field map, A2),
problem flash_forward: causal masking by comparing query and key positions.

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def main():
    rng = np.random.Generator(np.random.PCG64(20240601))
    n, d = 6, 4
    inp = {name: rng.standard_normal((n, d)) for name in ("q", "k", "v", "do")}
    scale = 0.5
    o, lse, _ = oracle.head_forward(inp["q"], inp["k"], inp["v"], True, scale)
    dq, dk, dv, _ = oracle.head_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, scale)
    fx = {
        "note": "oracle regression fixture; written by tests/golden/make_golden.py",
        "causal": True,
        "scale": scale,
        "inputs": {k: v.tolist() for k, v in inp.items()},
        "outputs": {"O": o.tolist(), "L": lse.tolist(), "dQ": dq.tolist(), "dK": dk.tolist(),
                    "dV": dv.tolist()},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_causal.json")
    with open(path, "w") as f:
        json.dump(fx, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
