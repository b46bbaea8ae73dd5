"""Writes tests/golden/oracle_small.json: a small seeded case with the fp64
oracle's outputs for both directions (regression fixture for the oracle; it
calls only oracle/ and the seeded input generator).

Operator: the triangle multiplicative update as the RFProteína architecture
page describes it ("Triangle multiplication on SM90", "Dual-GEMM gates"),
with the readings listed in the oracle module's docstring.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import tri_mul_intermediates  # noqa: E402
from pair_rep_triangle_amd.inputs import make_random  # noqa: E402


def main():
    d = make_random(1, 5, 4, 3, seed=2024, mask="random_pairs", random_affine=True)
    rec = {
        "source": "fp64 oracle (oracle/trimul_ref.py) via tests/golden/make_golden.py",
        "shape": {"batch": 1, "n": 5, "c_z": 4, "c": 3},
        "z": d["z"].astype(np.float64).tolist(),
        "mask": d["mask"].astype(np.float64).tolist(),
        "weights": {k: np.asarray(v, np.float64).tolist() for k, v in d["weights"].items()},
    }
    for direction in ("outgoing", "incoming"):
        it = tri_mul_intermediates(d["z"], d["mask"], d["weights"], direction)
        rec[direction] = {"x": it["x"].tolist(), "out": it["out"].tolist()}
    path = os.path.join(ROOT, "tests", "golden", "oracle_small.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
