"""Writes tests/golden/tiny_f32_oracle_rows.txt from the fp64 oracle alone.

The transcript prints no worked numeric example of this forward, so the only
stored expected values are this regression fixture: rows 0, 17, 40 and 63 of
the oracle's output on the seeded tiny workload (M=64, K=32, N=128, G=8,
eps=1e-5, seed 0).  It guards the oracle against unintended changes; the pins
in tests/oracle_pins.py are what tie the oracle to the method.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gemm_activation_groupnorm_amd.inputs import get_workload, workload_inputs  # noqa: E402

ROWS = (0, 17, 40, 63)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle_rows.txt")


def input_digest(inp):
    h = hashlib.sha256()
    for k in ("x", "W", "b_lin", "b_add", "gamma", "beta"):
        h.update(np.ascontiguousarray(inp[k], dtype=np.float32).tobytes())
    return h.hexdigest()


def main():
    w = get_workload("tiny_f32")
    inp = workload_inputs(w)
    y = oracle.lgn_forward(inp["x"], inp["W"], inp["b_lin"], inp["b_add"], inp["gamma"],
                           inp["beta"], w.G, w.eps)
    with open(OUT, "w") as f:
        f.write("# oracle output rows for workload %s (M=%d K=%d N=%d G=%d eps=%g seed=%d)\n"
                % (w.name, w.M, w.K, w.N, w.G, w.eps, w.seed))
        f.write("# written by tests/golden/make_golden.py (calls only oracle/)\n")
        f.write("input_sha256 %s\n" % input_digest(inp))
        for r in ROWS:
            f.write("row %d %s\n" % (r, " ".join(repr(float(v)) for v in y[r])))


if __name__ == "__main__":
    main()
