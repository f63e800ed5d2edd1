"""Write the oracle's per-row argmax of the output-head workload (K=5120, N=151936).

Calls only the CPU oracle (and the seeded input generator).  Rows are the 8 activation
rows of the seed-0 draw; a call with M rows uses the first M.  Run from the repo root:
    python tests/golden/make_head_argmax.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import argmax_rows, verify  # noqa: E402
from synthetic import workload_case  # noqa: E402

NAME = "head_affine2_k5120_n151936"


def main():
    case = workload_case(NAME, seed=0)
    y = verify(case.fmt, case.x(8), case.x_dtype, case.words, case.scales, case.biases)
    idx, gap = argmax_rows(y)
    out = {
        "workload": NAME, "seed": 0, "rows": 8,
        "argmax": [int(i) for i in idx],
        "top2_gap": [float(g) for g in gap],
        "row_absmax": [float(v) for v in abs(y).max(axis=1)],
        "note": "fp64 oracle: dequantize-then-matmul; argmax ties go to the lowest index",
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{NAME}_argmax.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path, out["argmax"], out["top2_gap"])


if __name__ == "__main__":
    main()
