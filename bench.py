#!/usr/bin/env python3
"""Benchmark of the fused Linear -> Swish -> +bias -> GroupNorm forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant fused|twopass] [--no-cpu-baseline] [--no-extra]

A step is one full forward (GEMM, bias, Swish, bias, GroupNorm statistics,
normalise, affine, output write) over one batch of seeded synthetic input that
is already resident in HBM.  W untimed warm-up steps, then K timed steps
bracketed by torch.cuda.synchronize().  Prints ONE JSON line on stdout; a
human-readable summary goes to stderr.

value      : GEMM TFLOP/s of the whole timed region, 2*M*N*K*K_steps / wall time.
roofline   : the fused kernel's mean time per launch from one HIP event pair
             recorded on the launch stream around the timed launches, against the MI355X
             dense MFMA peak of its input type (fp32 157.3, bf16 2500 TFLOP/s).
             traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
             counters (profiles/traffic.json), only if the kernel sources are
             unchanged since the counters were taken, else null.
cpu_baseline: the fp64 CPU oracle timed on the host on the first S rows of the
             same workload (S sized to about --cpu-seconds of work).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused Linear+Swish+bias+GroupNorm TFLOP/s at M32768 K1024 N4096; % MFMA peak"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "m32768_k1024_n4096_g64_f32"


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each variant's kernels are built from (a change to any of them
# voids that variant's stored counter values).
KERNEL_SOURCES = {
    "fused": ("lgn_device.hpp", "lgn_fused.hpp", "lgn_fused_impl.hpp", "lgn_fused_f32.hip",
              "lgn_fused_bf16.hip"),
    "twopass": ("lgn_device.hpp", "lgn_twopass.hpp", "lgn_twopass.hip"),
    "wide": ("lgn_device.hpp", "lgn_fused.hpp", "lgn_wide.hpp", "lgn_wide_impl.hpp",
             "lgn_wide_f32.hip", "lgn_wide_bf16.hip"),
    "lse": ("lgn_device.hpp", "lgn_lse.hpp", "lgn_lse.hip"),
    "lnconv": ("lgn_device.hpp", "lgn_sgh.hpp", "lgn_lnconv.hpp", "lgn_lnconv.hip"),
    "sgh": ("lgn_device.hpp", "lgn_sgh.hpp", "lgn_sgh.hip"),
}


def kernel_sources_sha(variant: str) -> str:
    # the build script counts too: it decides how the kernels are packaged
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_activation_groupnorm_amd", "csrc")
    files = [os.path.join(csrc, f) for f in KERNEL_SOURCES[variant]]
    files.append(os.path.join(ROOT, "gemm_activation_groupnorm_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(workload: str, variant: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get("%s/%s" % (workload, variant))
    if not rec or rec.get("src_sha") != kernel_sources_sha(variant):
        return None
    return rec.get("traffic_bytes")


class _Timed:
    """time(): W warm-up launches, then K timed ones on self.stream."""

    def time(self, steps: int, warmup: int, min_warm_ms: float = 0.0):
        """Wall time of `steps` back-to-back launches and the mean launch
        duration from one HIP event pair on the launch stream around them.
        `warmup` untimed launches first; with min_warm_ms > 0 the warm-up goes
        on until that much GPU time has passed (the clocks ramp up under load
        over tens of milliseconds)."""
        import torch
        t_warm = time.perf_counter()
        for _ in range(warmup):
            self.launch()
        torch.cuda.synchronize()
        while (time.perf_counter() - t_warm) * 1e3 < min_warm_ms:
            for _ in range(max(1, warmup)):
                self.launch()
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(self.stream)
        for _ in range(steps):
            self.launch()
        end.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, start.elapsed_time(end) / steps

    def distribution(self, launches: int = 50, flush_bytes: int = 0):
        """Per-launch durations (one HIP event pair around each launch on the
        launch stream): median, p10 and p90 in ms.  With flush_bytes > 0 a
        buffer of that size is overwritten between launches (outside the event
        pair), so that x and W no longer sit in L2 or MALL when a launch starts."""
        import numpy as np
        import torch
        buf = None
        if flush_bytes:
            buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device=self.out.device)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(launches)]
        with torch.cuda.stream(self.stream):
            for e0, e1 in pairs:
                if buf is not None:
                    buf.fill_(1.0)
                e0.record(self.stream)
                self.launch()
                e1.record(self.stream)
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in pairs])
        del buf
        return {"median_ms": round(float(np.median(ms)), 4),
                "p10_ms": round(float(np.percentile(ms, 10)), 4),
                "p90_ms": round(float(np.percentile(ms, 90)), 4)}

    def distributions(self, launches: int = 50):
        """Back-to-back and flushed (1 GiB overwritten between launches) per-launch timings."""
        hot = self.distribution(launches)
        cold = self.distribution(launches, flush_bytes=1 << 30)
        return {"launches": launches, **hot, "flushed_median_ms": cold["median_ms"],
                "flushed_p10_ms": cold["p10_ms"], "flushed_p90_ms": cold["p90_ms"],
                "flush_bytes": 1 << 30}


class Runner(_Timed):
    """Inputs resident on the GPU plus a launch() closure for one forward."""

    def __init__(self, w, variant: str):
        import numpy as np
        import torch
        from gemm_activation_groupnorm_amd import lgn
        from gemm_activation_groupnorm_amd.inputs import workload_inputs

        self.w, self.variant = w, variant
        t0 = time.perf_counter()
        self.inp = workload_inputs(w)
        dev = "cuda:0"
        self.d = {k: torch.from_numpy(np.ascontiguousarray(self.inp[k])).to(dev)
                  for k in ("b_lin", "b_add", "gamma", "beta")}
        if w.dtype == "bf16":
            for k in ("x", "W"):
                self.d[k] = torch.from_numpy(self.inp[k + "_bf16"].view(np.int16)).to(dev).view(
                    torch.bfloat16)
        else:
            for k in ("x", "W"):
                self.d[k] = torch.from_numpy(self.inp[k]).to(dev)
        self.ws = None
        if variant == "lse":
            self.out = torch.empty(w.M, dtype=torch.float32, device=dev)
            nb_lse = lgn.lgn_lse_workspace_bytes(w.M, w.N)
            self.ws = torch.empty(max(1, nb_lse // 4), dtype=torch.float32, device=dev)
        else:
            self.out = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        if variant == "twopass":
            self.ws = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        if variant == "wide":
            nb_wide = lgn.lgn_wide_workspace_bytes(w.M, w.N)
            self.ws = torch.empty(max(1, nb_wide // 4), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        eprint("[bench] %s/%s inputs ready in %.1f s" % (w.name, variant, time.perf_counter() - t0))
        self.stream = torch.cuda.current_stream()
        d, out = self.d, self.out
        args = (d["x"], d["W"], d["b_lin"], d["b_add"], d["gamma"], d["beta"],
                w.M, w.K, w.N, w.G, w.eps, out)
        s = self.stream
        if variant == "fused":
            fn = lgn.lgn_forward_f32 if w.dtype == "f32" else lgn.lgn_forward_bf16
            self.launch = lambda: lgn.check(fn(*args, stream=s))
        elif variant == "wide":
            fn = lgn.lgn_forward_wide_f32 if w.dtype == "f32" else lgn.lgn_forward_wide_bf16
            ws, nb_wide = self.ws, lgn.lgn_wide_workspace_bytes(w.M, w.N)
            self.launch = lambda: lgn.check(fn(*args, ws, nb_wide, stream=s))
        elif variant == "lse":
            fn = lgn.lgn_linear_lse_f32 if w.dtype == "f32" else lgn.lgn_linear_lse_bf16
            ws, nb_lse = self.ws, lgn.lgn_lse_workspace_bytes(w.M, w.N)
            lse_args = (d["x"], d["W"], d["b_lin"], w.M, w.K, w.N, out, ws, nb_lse)
            self.launch = lambda: lgn.check(fn(*lse_args, stream=s))
        else:
            fn = lgn.lgn_forward_twopass_f32 if w.dtype == "f32" else lgn.lgn_forward_twopass_bf16
            nb = lgn.lgn_twopass_workspace_bytes(w.M, w.N)
            ws = self.ws
            self.launch = lambda: lgn.check(fn(*args, ws, nb, stream=s))

    def check_rows(self, nrows: int = 8):
        import numpy as np
        import oracle
        from gemm_activation_groupnorm_amd.inputs import sample_rows
        rows = sample_rows(self.w.M, nrows, seed=99)
        import torch
        idx = torch.from_numpy(rows).to(self.out.device)
        y = self.out[idx].cpu().numpy().astype(np.float64)
        i = self.inp
        if self.variant == "lse":
            ref = oracle.linear_lse_forward(i["x"][rows], i["W"], i["b_lin"])
        else:
            ref = oracle.lgn_forward(i["x"][rows], i["W"], i["b_lin"], i["b_add"], i["gamma"],
                                     i["beta"], self.w.G, self.w.eps)
        return float(np.max(np.abs(y - ref))), len(rows)


class SghRunner(_Timed):
    """Swish -> spatial GroupNorm -> HardSwish on y [Nb, C, D*H*W], resident."""

    def __init__(self, w):
        import numpy as np
        import torch
        from gemm_activation_groupnorm_amd import lgn
        from gemm_activation_groupnorm_amd.inputs import make_sgh_inputs

        self.w, self.variant = w, "sgh"
        t0 = time.perf_counter()
        self.inp = make_sgh_inputs(w.Nb, w.C, w.S, w.seed)
        self.d = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0")
                  for k, v in self.inp.items()}
        self.out = torch.empty_like(self.d["y"])
        nb = lgn.lgn_sgh_workspace_bytes(w.Nb, w.C, w.S, w.G)
        self.ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        eprint("[bench] %s/sgh inputs ready in %.1f s" % (w.name, time.perf_counter() - t0))
        self.stream = torch.cuda.current_stream()
        d, s = self.d, self.stream
        args = (d["y"], d["gamma"], d["beta"], w.Nb, w.C, w.S, w.G, w.eps, self.out, self.ws, nb)
        self.launch = lambda: lgn.check(lgn.lgn_swish_gn_hardswish_f32(*args, stream=s))

    @property
    def algorithmic_bytes(self) -> int:
        """One read of y and one write of out (gamma, beta are 2*C floats)."""
        return 2 * self.w.elements * 4 + 2 * self.w.C * 4

    def check_rows(self, nrows: int = 2):
        """Max abs error against the oracle on `nrows` whole samples."""
        import numpy as np
        import oracle
        import torch
        from gemm_activation_groupnorm_amd.inputs import sample_rows
        rows = sample_rows(self.w.Nb, nrows, seed=99)
        y = self.out[torch.from_numpy(rows).to(self.out.device)].cpu().numpy().astype(np.float64)
        ref = oracle.swish_gn_hardswish(self.inp["y"][rows], self.inp["gamma"], self.inp["beta"],
                                        self.w.G, self.w.eps)
        return float(np.max(np.abs(y - ref))), len(rows)


class LnConvRunner(_Timed):
    """LayerNorm -> GELU -> dilated Conv1d -> + input on x [B, C, L], resident."""

    def __init__(self, w):
        import numpy as np
        import torch
        from gemm_activation_groupnorm_amd import lgn
        from gemm_activation_groupnorm_amd.inputs import make_lnconv_inputs

        self.w, self.variant = w, "lnconv"
        t0 = time.perf_counter()
        self.inp = make_lnconv_inputs(w.B, w.C, w.L, w.seed)
        self.d = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0")
                  for k, v in self.inp.items()}
        self.out = torch.empty_like(self.d["x"])
        nb = lgn.lgn_lnconv_workspace_bytes(w.B, w.C, w.L)
        self.ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        eprint("[bench] %s/lnconv inputs ready in %.1f s" % (w.name, time.perf_counter() - t0))
        self.stream = torch.cuda.current_stream()
        d, s = self.d, self.stream
        args = (d["x"], d["ln_w"], d["ln_b"], d["conv_w"], d["conv_b"], w.B, w.C, w.L, w.dilation,
                w.eps, w.gelu_tanh, self.out, self.ws, nb)
        self.launch = lambda: lgn.check(lgn.lgn_ln_gelu_conv1d_f32(*args, stream=s))

    def check_rows(self, ncols: int = 16):
        """Max abs error against the oracle on `ncols` sampled output columns (b, :, j)."""
        import numpy as np
        import oracle
        r = np.random.default_rng(99)
        w = self.w
        cols = [(int(b), int(j)) for b, j in zip(r.integers(0, w.B, ncols), r.integers(0, w.L, ncols))]
        ref = oracle.ln_gelu_conv1d_cols(self.inp["x"], self.inp["ln_w"], self.inp["ln_b"],
                                         self.inp["conv_w"], self.inp["conv_b"], w.dilation, w.eps,
                                         cols, gelu_tanh=w.gelu_tanh)
        y = np.stack([self.out[b, :, j].cpu().numpy() for b, j in cols]).astype(np.float64)
        return float(np.max(np.abs(y - ref))), len(cols)


def lnconv_main(args):
    """One JSON line for the LayerNorm -> GELU -> dilated Conv1d -> + input path
    (three launches per step), as convolution TFLOP/s."""
    from gemm_activation_groupnorm_amd.inputs import LNCONV_WORKLOADS
    w = [x for x in LNCONV_WORKLOADS if x.name == args.workload]
    if not w:
        raise SystemExit("--variant lnconv needs one of: %s" % [x.name for x in LNCONV_WORKLOADS])
    w = w[0]
    r = LnConvRunner(w)
    wall, kmean = r.time(args.steps, args.warmup)
    ach = w.flops / (kmean * 1e-3) / 1e12
    err, ncols = r.check_rows()
    eprint("[bench] %s/lnconv: %.3f ms/step, kernel mean %.3f ms -> %.1f TFLOP/s (%.1f%% of %.1f); "
           "sampled-column max err %.2e" % (w.name, wall / args.steps * 1e3, kmean, ach,
                                            100 * ach / PEAK_TFLOPS["f32"], PEAK_TFLOPS["f32"], err))
    print(json.dumps({
        "metric": "LayerNorm->GELU->dilated Conv1d->+x convolution TFLOP/s", "value": round(
            w.flops / (wall / args.steps) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "C": w.C, "L": w.L, "dilation": w.dilation,
                   "eps": w.eps, "gelu": "tanh" if w.gelu_tanh else "exact", "seed": w.seed,
                   "variant": "lnconv"},
        "roofline": {"bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_TFLOPS["f32"],
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS["f32"], 4),
                     "traffic": traffic_for(w.name, "lnconv"), "kernel_ms_mean": round(kmean, 4),
                     "kernel": "wpack+stats+lnconv"},
        "check": {"columns": ncols, "max_abs_err_vs_oracle": err}}), flush=True)


def torch_context(w):
    """Context only: torch's linear (vendor GEMM, output in the input type) and
    the unfused torch pipeline (linear, SiLU, add, group_norm) on random
    inputs of the workload's shape and type.  Not part of the product."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.randn(w.M, w.K, device="cuda", dtype=dt)
    W = torch.randn(w.N, w.K, device="cuda", dtype=dt)
    vec = [torch.randn(w.N, device="cuda") for _ in range(4)]

    def t(f, n=10):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def pipe():
        z = torch.nn.functional.linear(x, W).float() + vec[0]
        u = torch.nn.functional.silu(z) + vec[1]
        return torch.nn.functional.group_norm(u, w.G, vec[2], vec[3], w.eps)

    g_ms = t(lambda: torch.nn.functional.linear(x, W))
    p_ms = t(pipe)
    del x, W
    torch.cuda.empty_cache()
    return {"torch_linear_ms": round(g_ms, 4), "torch_linear_tflops": round(w.flops / g_ms / 1e9, 1),
            "torch_unfused_pipeline_ms": round(p_ms, 4),
            "note": "context only: torch linear = vendor GEMM with output in the input type"}


def cpu_baseline(w, inp, seconds: float):
    import oracle
    x, W = inp["x"], inp["W"]
    args = (inp["b_lin"], inp["b_add"], inp["gamma"], inp["beta"], w.G, w.eps)
    probe = min(w.M, 32)
    t0 = time.perf_counter()
    oracle.lgn_forward(x[:probe], W, *args)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(probe, min(w.M, seconds / max(per_row, 1e-9))))
    t0 = time.perf_counter()
    oracle.lgn_forward(x[:rows], W, *args)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "first %d of %d rows of %s, fp64 C oracle, %.1f s wall, %d OpenMP threads"
                  % (rows, w.M, w.name, dt, oracle.num_threads()),
    }


def sgh_main(args):
    """One JSON line for the HBM-bound Swish -> spatial GroupNorm -> HardSwish
    kernels (two launches per step), as GB/s of algorithmic traffic."""
    from gemm_activation_groupnorm_amd.inputs import SGH_WORKLOADS
    w = [x for x in SGH_WORKLOADS if x.name == args.workload]
    if not w:
        raise SystemExit("--variant sgh needs one of: %s" % [x.name for x in SGH_WORKLOADS])
    w = w[0]
    r = SghRunner(w)
    wall, kmean = r.time(args.steps, args.warmup)
    gbps = r.algorithmic_bytes / (kmean * 1e-3) / 1e9
    err, nrows = r.check_rows()
    eprint("[bench] %s/sgh: %.3f ms/step, kernel mean %.3f ms -> %.0f GB/s algorithmic (%.1f%% of "
           "%.0f); sampled-sample max err %.2e"
           % (w.name, wall / args.steps * 1e3, kmean, gbps, 100 * gbps / HBM_PEAK_GBPS,
              HBM_PEAK_GBPS, err))
    print(json.dumps({
        "metric": "Swish->spatial GroupNorm->HardSwish algorithmic HBM GB/s", "value": round(gbps, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "Nb": w.Nb, "C": w.C, "D": w.D, "H": w.H, "W": w.W,
                   "G": w.G, "eps": w.eps, "seed": w.seed, "variant": "sgh"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(w.name, "sgh"), "kernel_ms_mean": round(kmean, 4),
                     "kernel": "sgh stats+apply"},
        "check": {"samples": nrows, "max_abs_err_vs_oracle": err}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", default="fused",
                    choices=["fused", "twopass", "wide", "lse", "sgh", "lnconv"],
                    help="lse: Linear -> logsumexp -> LeakyReLU x2 -> GELU x2 (use with an "
                         "m1024_k8192_n8192_lse_* workload); sgh: Swish -> spatial GroupNorm -> "
                         "HardSwish (use with an *_sgh_* workload; reports GB/s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads (bf16, wide group, two-pass)")
    ap.add_argument("--no-per-launch", action="store_true",
                    help="skip the per-launch (median/p10/p90, flushed) timings, e.g. under a "
                         "profiler whose kernel averages should cover the timed launches only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--torch-context", action="store_true",
                    help="also time, for context only, torch's linear (vendor GEMM) and the "
                         "unfused torch pipeline on the same workload")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the forward, run the MFMA-ceiling probe (sustained MFMA rate "
                         "and shader clock for zero and random operands) and exit")
    ap.add_argument("--lds-bandwidth", action="store_true",
                    help="instead of the forward, run the LDS-bandwidth probe (16-byte LDS reads, "
                         "bytes per shader clock per CU) and exit")
    ap.add_argument("--l2-feed", action="store_true",
                    help="instead of the forward, run the operand-feed probe (global -> LDS DMA "
                         "of a 512-row panel with 64- or 128-byte LDS rows, bytes per shader "
                         "clock per CU) and exit")
    ap.add_argument("--fused-phases", action="store_true",
                    help="instead of the forward, run the fused-tile phase probe (shader cycles "
                         "of the main loop, epilogue and store drain per tile, and the clock) at "
                         "the pages' shape in bf16, and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the forward, run 5 plain device copies of MIB MiB (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the forward shards over rows (or whole groups) "
              "with no exchange, so a multi-GPU figure is N times the one-GPU figure on 1/N of "
              "the rows and is not run here (--gpus %d, WORLD_SIZE %d)." % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    if args.mfma_ceiling or args.lds_bandwidth or args.l2_feed or args.fused_phases:
        # a child process of its own: this process has not touched the GPU
        import subprocess
        from gemm_activation_groupnorm_amd import build as hip_build
        exe = (hip_build.PROBE if args.mfma_ceiling else
               hip_build.LDS_PROBE if args.lds_bandwidth else
               hip_build.FEED_PROBE if args.l2_feed else hip_build.PHASES_PROBE)
        if not os.path.exists(exe):
            hip_build.build_probe()
        sys.exit(subprocess.run([exe]).returncode)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "copies": 5}), flush=True)
        return
    from gemm_activation_groupnorm_amd import build as hip_build
    if not os.path.exists(hip_build.LIB):
        hip_build.build()
    from gemm_activation_groupnorm_amd.inputs import get_workload

    if args.variant == "sgh":
        sgh_main(args)
        return
    if args.variant == "lnconv":
        lnconv_main(args)
        return
    w = get_workload(args.workload)
    r = Runner(w, args.variant)
    wall, kmean = r.time(args.steps, args.warmup)
    flops = float(w.flops)
    ms_per_step = wall / args.steps * 1e3
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kmean * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    dist = None if args.no_per_launch else r.distributions()
    err, nrows = r.check_rows()
    if dist:
        eprint("[bench] %s/%s per launch: median %.3f ms (p10 %.3f, p90 %.3f); flushed median "
               "%.3f ms" % (w.name, args.variant, dist["median_ms"], dist["p10_ms"], dist["p90_ms"],
                            dist["flushed_median_ms"]))
    eprint("[bench] %s/%s: %.3f ms/step, kernel mean %.3f ms -> %.1f TFLOP/s (%.1f%% of %.1f); "
           "sampled-row max err %.2e"
           % (w.name, args.variant, ms_per_step, kmean, achieved, 100 * achieved / peak, peak, err))
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "G": w.G, "eps": w.eps,
                   "seed": w.seed, "variant": args.variant,
                   "inputs": "x~%g*N(0,1); W,b_lin~U(+-1/sqrt(K)); b_add~0.02*N(0,1); "
                             "gamma~1+0.1*N(0,1); beta~0.1*N(0,1)" % w.x_scale},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic_for(w.name, args.variant),
            "kernel_ms_mean": round(kmean, 4),
            "kernel": {"fused": "lgn_fused_kernel", "twopass": "gemm+epilogue",
                       "wide": "wide partial+norm", "lse": "lse partial+finish"}[args.variant],
        },
        "per_launch": dist,
        "check": {"rows": nrows, "max_abs_err_vs_oracle": err},
    }
    inp = r.inp
    del r
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = []
        for name, variant in (("m32768_k1024_n4096_g64_bf16", "fused"),
                              ("m16384_k2048_n8192_g8_f32", "fused"),
                              (DEFAULT_WORKLOAD, "twopass"),
                              ("m32768_k1024_n4096_g64_bf16", "twopass"),
                              ("m16384_k2048_n8192_g8_f32", "twopass"),
                              ("m16384_k2048_n8192_g8_f32", "wide"),
                              ("m16384_k2048_n8192_g1_f32", "wide"),
                              ("m1024_k8192_n8192_lse_f32", "lse"),
                              ("m1024_k8192_n8192_lse_bf16", "lse")):
            if name == w.name and variant == args.variant:
                continue
            we = get_workload(name)
            re = Runner(we, variant)
            n_extra = 50
            wl, km_mean = re.time(n_extra, 5, min_warm_ms=100.0)
            ach = we.flops / (km_mean * 1e-3) / 1e12
            dist_e = re.distributions() if (variant == "fused" and we.dtype == "bf16") else None
            e2, _ = re.check_rows(4)
            eprint("[bench] %s/%s: kernel mean %.3f ms -> %.1f TFLOP/s (%.1f%% of %.1f), err %.2e"
                   % (name, variant, km_mean, ach, 100 * ach / PEAK_TFLOPS[we.dtype],
                      PEAK_TFLOPS[we.dtype], e2))
            extra.append({"workload": name, "variant": variant, "dtype": we.dtype,
                          "ms_per_step": round(wl / n_extra * 1e3, 4), "kernel_ms_mean": round(km_mean, 4),
                          "tflops": round(ach, 3), "frac_of_peak": round(ach / PEAK_TFLOPS[we.dtype], 4),
                          "max_abs_err_vs_oracle": e2})
            if dist_e:
                extra[-1]["per_launch"] = dist_e
            del re
            torch.cuda.empty_cache()
        from gemm_activation_groupnorm_amd.inputs import SGH_WORKLOADS
        for ws_ in SGH_WORKLOADS:
            if args.variant == "sgh":
                continue
            rs = SghRunner(ws_)
            n_extra = 30
            wl, km_mean = rs.time(n_extra, 3, min_warm_ms=100.0)
            gbps = rs.algorithmic_bytes / (km_mean * 1e-3) / 1e9
            e2, _ = rs.check_rows(2)
            eprint("[bench] %s/sgh: kernel mean %.3f ms -> %.0f GB/s algorithmic (%.1f%% of %.0f), "
                   "err %.2e" % (ws_.name, km_mean, gbps, 100 * gbps / HBM_PEAK_GBPS, HBM_PEAK_GBPS,
                                 e2))
            extra.append({"workload": ws_.name, "variant": "sgh", "dtype": "f32",
                          "ms_per_step": round(wl / n_extra * 1e3, 4),
                          "kernel_ms_mean": round(km_mean, 4), "algorithmic_gbps": round(gbps, 1),
                          "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                          "max_abs_err_vs_oracle": e2})
            del rs
            torch.cuda.empty_cache()
        from gemm_activation_groupnorm_amd.inputs import LNCONV_WORKLOADS
        for wl_ in LNCONV_WORKLOADS:
            rl = LnConvRunner(wl_)
            n_extra = 30
            wl, km_mean = rl.time(n_extra, 3, min_warm_ms=100.0)
            ach = wl_.flops / (km_mean * 1e-3) / 1e12
            e2, _ = rl.check_rows(8)
            eprint("[bench] %s/lnconv: kernel mean %.3f ms -> %.1f TFLOP/s (%.1f%% of %.1f), "
                   "err %.2e" % (wl_.name, km_mean, ach, 100 * ach / PEAK_TFLOPS["f32"],
                                 PEAK_TFLOPS["f32"], e2))
            extra.append({"workload": wl_.name, "variant": "lnconv", "dtype": "f32",
                          "ms_per_step": round(wl / n_extra * 1e3, 4),
                          "kernel_ms_mean": round(km_mean, 4), "tflops": round(ach, 3),
                          "frac_of_peak": round(ach / PEAK_TFLOPS["f32"], 4),
                          "max_abs_err_vs_oracle": e2})
            del rl
            torch.cuda.empty_cache()
        res["extra"] = extra

    if args.torch_context:
        res["torch_context"] = torch_context(w)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
        eprint("[bench] cpu baseline: %s" % res["cpu_baseline"]["sample"])
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
