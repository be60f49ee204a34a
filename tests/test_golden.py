"""The oracle reproduces its stored output on the seeded tiny workload
(regression fixture written by tests/golden/make_golden.py)."""
import os

import numpy as np

import oracle
from gemm_activation_groupnorm_amd.inputs import get_workload, workload_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _read():
    rows, digest = {}, None
    with open(os.path.join(HERE, "golden", "tiny_f32_oracle_rows.txt")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "input_sha256":
                digest = parts[1]
            elif parts[0] == "row":
                rows[int(parts[1])] = np.array([float(v) for v in parts[2:]])
    return digest, rows


def test_tiny_inputs_unchanged():
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden
    digest, _ = _read()
    assert make_golden.input_digest(workload_inputs(get_workload("tiny_f32"))) == digest


def test_oracle_reproduces_golden_rows():
    w = get_workload("tiny_f32")
    inp = workload_inputs(w)
    y = oracle.lgn_forward(inp["x"], inp["W"], inp["b_lin"], inp["b_add"], inp["gamma"],
                           inp["beta"], w.G, w.eps)
    _, rows = _read()
    assert len(rows) == 4
    for r, ref in rows.items():
        np.testing.assert_allclose(y[r], ref, rtol=0, atol=1e-14)
