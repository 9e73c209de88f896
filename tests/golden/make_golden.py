"""Write tests/golden/tiny_oracle.json from the CPU oracle only.

The fixture is a regression record of the oracle on the tiny workload
(T=16, hidden 256, 8 experts, top-2, FFN 128, no shared expert; seed 0):
routing, grouping and a digest of y.  It is written by this script, which
calls nothing but the oracle and the seeded input generator, so that any
later change to the oracle's arithmetic shows up as a changed fixture.

    python -m tests.golden.make_golden
"""
import json
import os

import numpy as np

import oracle
from sparse_moe_layer_03_amd import synth

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")


def record():
    inp = synth.make_inputs("tiny", seed=0)
    r = oracle.forward(inp)
    counts, offsets, perm = oracle.align(r["ids"], inp["wl"].E)
    y = r["y"]
    return {
        "workload": inp["wl"].note,
        "seed": 0,
        "input_hash": synth.content_hash(inp),
        "ids": r["ids"].tolist(),
        "w": [[float(v) for v in row] for row in r["w"]],
        "counts": counts.tolist(),
        "perm": perm.tolist(),
        "y_row0_first8": [float(v) for v in y[0, :8]],
        "y_row_l2": [float(v) for v in np.linalg.norm(y, axis=1)],
        "y_sum": float(y.sum()),
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(record(), f, indent=1)
    print("wrote", OUT)
