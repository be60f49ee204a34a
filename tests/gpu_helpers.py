"""Helpers for the GPU tests: move seeded inputs to the device, call the C ABI
through the binding, and compare against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import make_inputs

TOL = {"f32": 2e-4, "bf16": 3e-2}
DEV = "cuda:0"


def log(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a crash log says where."""
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def to_device(inp: dict, dtype: str) -> dict:
    d = {}
    for k in ("b_lin", "b_add", "gamma", "beta"):
        d[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(DEV)
    if dtype == "bf16":
        for k in ("x", "W"):
            bits = np.ascontiguousarray(inp[k + "_bf16"]).view(np.int16)
            d[k] = torch.from_numpy(bits).to(DEV).view(torch.bfloat16)
    else:
        for k in ("x", "W"):
            d[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(DEV)
    return d


def run(dev: dict, M, K, N, G, eps, dtype="f32", variant="fused", out=None, ws=None,
        stream=None):
    """Call one entry point; returns the output tensor (status checked)."""
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=DEV)
    args = (dev["x"], dev["W"], dev["b_lin"], dev["b_add"], dev["gamma"], dev["beta"],
            M, K, N, G, eps, out)
    if variant == "fused":
        fn = lgn.lgn_forward_f32 if dtype == "f32" else lgn.lgn_forward_bf16
        st = fn(*args, stream=stream)
    else:
        fn = lgn.lgn_forward_twopass_f32 if dtype == "f32" else lgn.lgn_forward_twopass_bf16
        if ws is None:
            ws = torch.empty(max(1, M * N), dtype=torch.float32, device=DEV)
        st = fn(*args, ws, lgn.lgn_twopass_workspace_bytes(M, N), stream=stream)
    lgn.check(st)
    return out


def oracle_rows(inp: dict, G: int, eps: float, rows=None) -> np.ndarray:
    x = inp["x"] if rows is None else inp["x"][rows]
    return oracle.lgn_forward(x, inp["W"], inp["b_lin"], inp["b_add"], inp["gamma"],
                              inp["beta"], G, eps)


def max_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    assert y_gpu.shape == y_ref.shape
    if y_gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(y_gpu)), "non-finite GPU output"
    return float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref)))


def case(M, K, N, G, seed, dtype="f32", x_scale=1.0):
    return make_inputs(M, K, N, seed, dtype, x_scale)


class ErrStats:
    """Running error statistics of GPU output against the fp64 oracle over
    every compared element: max abs, mean abs, and the count above the
    tolerance.  Non-finite GPU values fail at once."""

    def __init__(self, tol: float):
        self.tol = tol
        self.max = 0.0
        self.sum = 0.0
        self.n = 0
        self.over = 0

    def add(self, y_gpu: np.ndarray, y_ref: np.ndarray) -> None:
        assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
        if y_gpu.size == 0:
            return
        assert np.all(np.isfinite(y_gpu)), "non-finite GPU output"
        d = np.abs(y_gpu.astype(np.float64) - y_ref)
        self.max = max(self.max, float(d.max()))
        self.sum += float(d.sum())
        self.n += d.size
        self.over += int(np.count_nonzero(d > self.tol))

    @property
    def mean(self) -> float:
        return self.sum / self.n if self.n else 0.0

    def summary(self) -> dict:
        return {"elements": self.n, "max_abs": self.max, "mean_abs": self.mean,
                "count_gt_tol": self.over, "tol": self.tol}

    def __str__(self) -> str:
        return ("max abs %.3e, mean abs %.3e, %d of %d elements > %.0e"
                % (self.max, self.mean, self.over, self.n, self.tol))


def compare_all_rows(outputs: dict, oracle_chunk, rows: int, tol: float,
                     chunk: int = 2048) -> dict:
    """Every element of each GPU output (host arrays whose first axis is the
    row) against the oracle, computed once per chunk of rows:
    oracle_chunk(r0, r1) returns the fp64 rows r0..r1-1.  Returns
    {name: ErrStats}."""
    stats = {k: ErrStats(tol) for k in outputs}
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        ref = oracle_chunk(r0, r1)
        for k, y in outputs.items():
            stats[k].add(y[r0:r1], ref)
    return stats
