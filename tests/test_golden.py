"""The fp64 oracle still reproduces its frozen tiny-configuration output."""
import json
import os

import numpy as np

from recurrent_cell_amd.inputs import CONFIGS, cfc_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cfc_tiny_seed0.json")


def test_oracle_matches_frozen_tiny_output(oracle_mod):
    with open(GOLDEN) as f:
        g = json.load(f)
    x = cfc_inputs(**CONFIGS["tiny"], seed=0)
    r = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64")
    assert abs(r["loss"] - g["loss"]) <= 1e-12 * abs(g["loss"])
    np.testing.assert_allclose(r["h_hist"][-1, 0], g["h_K_sample0"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["gb"], g["gb"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["gW"][0, 0], g["gW_f_row0"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dh0"][0], g["dh0_sample0"], rtol=1e-12, atol=1e-14)
    assert abs(np.abs(r["gW"]).sum() - g["gW_abs_sum"]) <= 1e-12 * g["gW_abs_sum"]
