"""Writes tests/golden/oracle_tiny.json: the fp64 oracle's results on the
tiny workload (B1 H1 N1024 D64, block 64, 50% sparsity, seeded inputs), as a
regression fixture for the oracle itself.

No page prints a worked example of BA-Att (the BA-Att review's referee report
asks for pseudocode of the norm sort), so no stored value here comes from the
pages: every value is the oracle's, written by this script, which calls only
oracle/ and the seeded input generator.  A later change of the oracle's
arithmetic shows up as a failing pin and must name, in its commit message, the
passage or reading that justifies it.

    python tests/golden/make_oracle_golden.py
"""

import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from block_sparse_attention_ba_amd import workloads  # noqa: E402  (seeded inputs only)
from oracle import ba_att_oracle as orc  # noqa: E402

ROWS = [0, 1, 63, 64, 500, 1023]  # query rows whose outputs are stored


def compute():
    x = workloads.make_inputs("tiny")
    w = x["workload"]
    sp = 0.5
    sel = orc.select_oracle(x["q"], x["k"], w.block, sp)
    att = orc.attention_oracle(x["q"], x["k"], x["v"], sel["mask"], w.block)
    O, L = att[(0, 0)]
    return {
        "workload": "tiny: B1 H1 N1024 D64, block 64, sparsity 0.5, scale 1/sqrt(64)",
        "keep": int(sel["keep"]),
        "S": sel["S"][0, 0].tolist(),
        "mask": sel["mask"][0, 0].tolist(),
        "idx": sel["idx"][0, 0].tolist(),
        "lse": [float(v) for v in L],
        "o_rows": {str(r): [float(v) for v in O[r]] for r in ROWS},
        "scale": 1.0 / math.sqrt(w.D),
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=None, separators=(",", ":"))
    print("wrote", out)
