"""The oracle's result on the tiny workload matches its frozen golden file."""
import os

import numpy as np

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.txt")


def test_tiny_golden():
    rows = {"out": {}, "last": {}}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#"):
                continue
            kind, idx, *vals = line.split()
            rows[kind][int(idx)] = np.array([float(v) for v in vals])
    w = WORKLOADS["tiny"]
    t = make_inputs(w)
    out, last = orc.selective_scan(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                   t["z"], t["delta_bias"], True, io_dtype=w.io_dtype)
    want_out = np.stack([rows["out"][i] for i in range(len(rows["out"]))])
    want_last = np.stack([rows["last"][i] for i in range(len(rows["last"]))])
    np.testing.assert_allclose(out, want_out, rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(last, want_last, rtol=1e-15, atol=1e-300)
