"""Writes tests/golden/tiny_oracle.txt: the oracle's output on the 'tiny'
workload (b=1, d=16, l=64, n=4, fp32, seed 0).

The pages print no worked numbers for the selective scan, so this file is not
a value from the pages: it freezes the oracle's own result so that any later
change to the oracle's arithmetic shows up as a diff.  It calls only oracle/
and the seeded input generator.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as orc  # noqa: E402
from state_space_model_scan_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")


def main():
    w = WORKLOADS["tiny"]
    t = make_inputs(w)
    out, last = orc.selective_scan(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                   t["z"], t["delta_bias"], True, io_dtype=w.io_dtype)
    with open(OUT, "w") as f:
        f.write("# oracle output, workload tiny (b=1 d=16 l=64 n=4 fp32 seed 0)\n")
        f.write("# written by tests/golden/make_golden.py; rows: out[d, t] then last_state[d, s]\n")
        for r in range(out.shape[0]):
            f.write("out %d " % r + " ".join("%.17g" % v for v in out[r]) + "\n")
        for r in range(last.shape[0]):
            f.write("last %d " % r + " ".join("%.17g" % v for v in last[r]) + "\n")


if __name__ == "__main__":
    main()
