"""Write tests/golden/config1_oracle.json from the oracle alone.

Workload 1 (one 64x64 fp32 matrix, 64-point Hadamard, K=2, fixed scale 1.0):
packed words, the tail-biting end state X and the bit pattern of each tile's
squared error.  Only the oracle and the seeded input generator are used.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    m = workloads.config(1)[0]
    out = oracle.quantize_matrix(m.w, m.su, m.sv, m.K, had_block=m.had_block, gss=None,
                                 fixed_scale=1.0)
    g = {
        "_about": "oracle output for workload 1, written by tests/golden/make_golden.py",
        "packed": out["packed"].astype(np.int64).ravel().tolist(),
        "X": [int(x) for x in out["X"]],
        "sse_bits": out["sse"].view(np.uint32).tolist(),
        "mse": out["mse"],
    }
    with open(os.path.join(HERE, "config1_oracle.json"), "w") as f:
        json.dump(g, f)
    print("mse", out["mse"])


if __name__ == "__main__":
    main()
