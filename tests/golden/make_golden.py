"""Write the stored oracle outputs under tests/golden/.

Calls only the CPU oracle (``oracle``) on inputs from the seeded workload
generator; nothing here comes from the GPU path.  Run from the repository
root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from long_context_biased_amd import workloads  # noqa: E402

#: query positions stored per case: tile and bias-cell edges, the end.
ROWS = [0, 15, 16, 63, 64, 200, 511]


def tiny_case(hot):
    L = workloads.make_layer("tiny", hot=hot)
    bias = oracle.project_pair_bias(L.pair, L.weight)
    out = oracle.attention_rows(L.q, L.k, L.v, bias, ROWS, scale=L.scale, cap=L.cap)
    return {
        "workload": "tiny" + ("_hot" if hot else ""),
        "source": "oracle.attention_rows on workloads.make_layer('tiny', hot=%s)" % hot,
        "rows": ROWS,
        "dv": list(range(8)),
        # out[row][head][dv] for the first 8 value channels
        "out": np.round(out[:, :, :8], 17).tolist(),
        "row_sums": np.round(out.sum(axis=-1), 17).tolist(),
    }


def main():
    cases = [tiny_case(False), tiny_case(True)]
    with open(os.path.join(HERE, "tiny_oracle_rows.json"), "w") as f:
        json.dump({"note": "Float64 oracle outputs (regression fixture).",
                   "cases": cases}, f, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
