"""Writes tests/golden/tiny_oracle.json from the oracle alone.

The pages print no worked numeric example for this path, so the only stored
values are the oracle's own, on the tiny workload (B=1, 2 heads, d=32, K=4,
conv width 4 over 192 channels, fp32, seed 0).  The fixture pins the oracle
against unnoticed drift: a later change to its arithmetic must regenerate
this file and say why.  Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from speculative_verify_gdn_amd import synth  # noqa: E402


def compute():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl, seed=0)
    x = inp["x"].float().numpy()
    w = inp["w"].numpy()
    hist = inp["hist"].float().numpy()
    y, hist_out, win = oracle.conv_step_f32(x, w, hist, round_bf16=False)
    f = lambda k: inp[k].double().numpy()
    S_out, H, o = oracle.gdn_recurrent_f64(y, f("beta_raw"), f("alpha"), f("dt_bias"), f("A_log"),
                                           f("S_in"), wl.Hk)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, S_out.size, 64)
    hidx = rng.integers(0, H.size, 64)
    return {
        "workload": wl.as_dict(),
        "seed": 0,
        "y_f32_hex": [float(v).hex() for v in y.reshape(-1)],
        "o": [float(v) for v in o.reshape(-1)],
        "S_out_idx": [int(i) for i in idx],
        "S_out_vals": [float(v) for v in S_out.reshape(-1)[idx]],
        "H_idx": [int(i) for i in hidx],
        "H_vals": [float(v) for v in H.reshape(-1)[hidx]],
        "S_out_fro": float(np.linalg.norm(S_out)),
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(out, "w") as fh:
        json.dump(compute(), fh, indent=0)
    print("wrote", out)
