"""Write tests/golden/cfc_tiny_seed0.json from the CPU oracle alone.

The pages print no worked numeric example of the cell, so this fixture is not
a pin of correctness: it freezes the fp64 oracle's output on the tiny
configuration (B=4, C=16, n_x=8, K=4, seed 0, zero biases) so that any later
change to the oracle's arithmetic shows up as a diff that its commit must
justify.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from recurrent_cell_amd.inputs import CONFIGS, cfc_inputs  # noqa: E402


def main():
    x = cfc_inputs(**CONFIGS["tiny"], seed=0)
    r = oracle.train(x.u, x.y, x.h0, x.W, x.bias, "f64")
    doc = {
        "source": "oracle fp64, tiny configuration B=4 C=16 n_x=8 K=4, inputs seed 0",
        "loss": r["loss"],
        "h_K_sample0": r["h_hist"][-1, 0].tolist(),
        "gb": r["gb"].tolist(),
        "gW_f_row0": r["gW"][0, 0].tolist(),
        "gW_sum": float(r["gW"].sum()),
        "gW_abs_sum": float(np.abs(r["gW"]).sum()),
        "dh0_sample0": r["dh0"][0].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfc_tiny_seed0.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
