"""Writes tests/golden/tiny_oracle.json from the oracle alone.

The MAGE page prints no worked example with intermediate values, so the only
stored values are regression fixtures of the oracle itself on the seeded
``tiny`` workload (1 seq, 1/1 heads, d=64, N=1024, B=16, k=64), written by
this script, which calls only ``oracle`` and the input generator.

    python tests/golden/make_golden.py
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
    inp = workloads.make_inputs(0)
    w = inp.w
    O, lse, sc, idx = oracle.select_exact(inp.q1, inp.k, inp.v, w.scale, w.k)
    Os, lses = oracle.sparse(inp.q_steps[0], inp.k, inp.v, idx, w.scale)
    out = {
        "workload": "tiny (seed 1000): 1 seq, 1/1 heads, d=64, N=1024, B=16, k=64, scale 0.125",
        "idx": idx[0, 0].tolist(),
        "lse_step1": lse[0, :, 0].tolist(),
        "o_step1_row_sums": O[0, :, 0].sum(-1).tolist(),
        "score_top8": sorted(sc[0][0].tolist(), reverse=True)[:8],
        "lse_step2": lses[0, :, 0].tolist(),
        "o_step2_row_sums": Os[0, :, 0].sum(-1).tolist(),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
