"""The oracle still reproduces its stored tiny-workload outputs.

tests/golden/tiny_oracle.json was written by tests/golden/make_golden.py,
which calls only the oracle.  The conv output is compared bit for bit, the
double-precision GDN outputs to 1e-14.
"""
import json
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_stored_tiny_outputs():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    ref = json.load(open(path))
    now = make_golden.compute()
    assert now["workload"] == ref["workload"]
    assert now["y_f32_hex"] == ref["y_f32_hex"]
    assert np.allclose(now["o"], ref["o"], rtol=0, atol=1e-14)
    assert now["S_out_idx"] == ref["S_out_idx"] and now["H_idx"] == ref["H_idx"]
    assert np.allclose(now["S_out_vals"], ref["S_out_vals"], rtol=0, atol=1e-14)
    assert np.allclose(now["H_vals"], ref["H_vals"], rtol=0, atol=1e-14)
