#!/usr/bin/env python3
"""Benchmark of the fused Linear -> Swish -> +bias -> GroupNorm forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant fused|twopass|wide|lse|sgh|lnconv]
                    [--no-cpu-baseline] [--no-extra]

A step is one full forward (GEMM, bias, Swish, bias, GroupNorm statistics,
normalise, affine, output write) over one batch of seeded synthetic input that
is already resident in HBM.  W untimed warm-up steps, then K timed steps
bracketed by torch.cuda.synchronize().  Prints ONE JSON line on stdout; a
human-readable summary goes to stderr.

value      : GEMM TFLOP/s of the whole timed region, 2*M*N*K*K_steps / wall time.
roofline   : the kernel's mean time per launch from one HIP event pair recorded
             on the launch stream around the timed launches, against the MI355X
             dense MFMA peak of its input type (fp32 157.3, bf16 2500 TFLOP/s);
             frac_at_sclk divides by that peak scaled to the median shader
             clock of the timed region (the peaks are quoted at 2400 MHz).
             traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
             counters (profiles/traffic.json), only if the kernel sources are
             unchanged since the counters were taken, else null.
extra      : the other workloads and entry points, timed the same way.
telemetry  : the GPU's shader clock and board power sampled from sysfs during
             the timed regions, and the host CPU model.
cpu_baseline: the fp64 CPU oracle, built for this host, timed on the first S
             rows of the workload (S sized to about --cpu-seconds of work).
             The same leg computes the oracle over EVERY element of every
             timed output and reports, per line, max abs, mean abs and the
             count above the tolerance ("check").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import tempfile
import threading
import time
from typing import Optional

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused Linear+Swish+bias+GroupNorm TFLOP/s at M32768 K1024 N4096; % MFMA peak"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
HBM_PEAK_GBPS = 8000.0
PEAK_SCLK_MHZ = 2400.0      # the shader clock the MFMA peaks are quoted at
TOL = {"f32": 2e-4, "bf16": 3e-2}
DEFAULT_WORKLOAD = "m32768_k1024_n4096_g64_f32"


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each variant's kernels are built from (a change to any of them
# voids that variant's stored counter values).
KERNEL_SOURCES = {
    # the fused entry point runs the two-pass kernels for fp32 groups of 512
    # or more channels, and its dispatch lives in lgn_api.hip / lgn_launch.hpp
    "fused": ("lgn_device.hpp", "lgn_fused.hpp", "lgn_fused.hip", "lgn_launch.hpp",
              "lgn_api.hip", "lgn_twopass.hpp", "lgn_twopass.hip"),
    "twopass": ("lgn_device.hpp", "lgn_twopass.hpp", "lgn_twopass.hip"),
    "wide": ("lgn_device.hpp", "lgn_fused.hpp", "lgn_wide.hpp", "lgn_wide.hip"),
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


def sha256s(arrays: dict) -> dict:
    """SHA-256 of each input array's bytes (the exact values both sides see)."""
    import numpy as np
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
            for k, v in sorted(arrays.items())}


# ------------------------------------------------------------ telemetry ----

def host_info() -> dict:
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:   # lscpu missing: fall back to /proc/cpuinfo
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


class Telemetry:
    """Samples the GPU's shader clock (amdgpu hwmon freq1_input labelled
    "sclk") and board power (hwmon power1_average or power1_input) from sysfs
    every `interval` seconds in a background thread, and summarises the
    samples that fall inside each named window (the timed regions)."""

    def __init__(self, interval: float = 0.01):
        self.interval = interval
        self.samples = []          # (t, sclk_mhz or None, power_w or None)
        self.windows = {}          # name -> (t0, t1)
        self.source = None
        self._stop = threading.Event()
        self._thread = None
        self._sclk, self._power = self._find()

    def _find(self):
        try:
            import torch
            p = torch.cuda.get_device_properties(0)
            pci = "%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
        except Exception as e:   # no device properties: nothing to sample
            self.source = "unavailable (%s)" % e
            return None, None
        hw = os.path.join("/sys/bus/pci/devices", pci, "hwmon")
        sclk = power = None
        if os.path.isdir(hw):
            for d in sorted(os.listdir(hw)):
                dd = os.path.join(hw, d)
                try:
                    with open(os.path.join(dd, "freq1_label")) as f:
                        if f.read().strip() == "sclk":
                            sclk = os.path.join(dd, "freq1_input")
                except OSError:
                    pass
                for f in ("power1_average", "power1_input"):
                    if power is None and os.path.exists(os.path.join(dd, f)):
                        power = os.path.join(dd, f)
        if sclk is None:
            # no hwmon clock: the current DPM level of pp_dpm_sclk ("N: 2100Mhz *")
            dpm = os.path.join("/sys/bus/pci/devices", pci, "pp_dpm_sclk")
            if os.path.exists(dpm):
                sclk = dpm
        cap = self._read(os.path.join(os.path.dirname(power), "power1_cap"), 1e-6) if power else None
        self.source = {"pci": pci, "sclk": sclk, "power": power, "power_cap_w": cap}
        return sclk, power

    @staticmethod
    def _read(path, scale):
        if path is None:
            return None
        try:
            with open(path) as f:
                text = f.read()
            if path.endswith("pp_dpm_sclk"):
                for line in text.splitlines():
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("M")[0].split("m")[0])
                return None
            return int(text.strip()) * scale
        except (OSError, ValueError, IndexError):
            return None

    def _run(self):
        while not self._stop.is_set():
            self.samples.append((time.perf_counter(), self._read(self._sclk, 1e-6),
                                 self._read(self._power, 1e-6)))
            self._stop.wait(self.interval)

    def start(self):
        if self._sclk or self._power:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def window(self, name, t0, t1):
        self.windows[name] = (t0, t1)

    def summary(self, name):
        if name not in self.windows:
            return None
        t0, t1 = self.windows[name]
        sel = [s for s in self.samples if t0 <= s[0] <= t1]
        out = {"samples": len(sel)}
        for i, key in ((1, "sclk_mhz"), (2, "power_w")):
            v = sorted(s[i] for s in sel if s[i] is not None)
            if v:
                out[key] = {"min": round(v[0], 1), "median": round(v[len(v) // 2], 1),
                            "max": round(v[-1], 1)}
        return out


MIN_CLOCK_SAMPLES = 5


def frac_at_clock(achieved: float, peak: float, telemetry) -> Optional[float]:
    """achieved / (peak scaled to the median shader clock of the timed
    region), or None without at least MIN_CLOCK_SAMPLES clock readings or
    while the readings still move by more than 10 % (the sysfs clock level
    trails a GPU that has just left idle)."""
    try:
        clk = telemetry["sclk_mhz"]
        mhz, n = clk["median"], telemetry["samples"]
    except (TypeError, KeyError):
        return None
    if not mhz or n < MIN_CLOCK_SAMPLES or (clk["max"] - clk["min"]) > 0.1 * mhz:
        return None
    return round(achieved / (peak * mhz / PEAK_SCLK_MHZ), 4)


# --------------------------------------------------------------- timing ----

class _Timed:
    """time(): W warm-up launches, then K timed ones on self.stream."""

    def time(self, steps: int, warmup: int, min_warm_ms: float = 0.0):
        """Wall time of `steps` back-to-back launches and the mean launch
        duration from one HIP event pair on the launch stream around them.
        `warmup` untimed launches first; with min_warm_ms > 0 the warm-up goes
        on until that much GPU time has passed (the clocks ramp up under load
        over tens of milliseconds).  Returns (wall, mean_ms, t0, t1, w0):
        [t0, t1] is the timed region, w0 the start of the warm-up's last
        100 ms (the same launches), for telemetry when the timed region alone
        holds too few sysfs samples."""
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
        t1 = time.perf_counter()
        return t1 - t0, start.elapsed_time(end) / steps, t0, t1, max(t_warm, t0 - 0.1)

    def distribution(self, launches: int = 50, flush_bytes: int = 0):
        """Per-launch durations (one HIP event pair around each launch on the
        launch stream): median, p10 and p90 in ms.  With flush_bytes > 0 a
        buffer of that size is overwritten between launches (outside the event
        pair), so that the inputs no longer sit in L2 or MALL when a launch starts."""
        import numpy as np
        import torch
        buf = None
        if flush_bytes:
            buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda:0")
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

    def host_output(self):
        """The output of the last launch, copied to host memory."""
        import torch
        torch.cuda.synchronize()
        return self.out.cpu().numpy()


def gemm_device_inputs(w, inp):
    import numpy as np
    import torch
    dev = "cuda:0"
    d = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
         for k in ("b_lin", "b_add", "gamma", "beta")}
    for k in ("x", "W"):
        if w.dtype == "bf16":
            d[k] = torch.from_numpy(inp[k + "_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            d[k] = torch.from_numpy(inp[k]).to(dev)
    return d


class Runner(_Timed):
    """One entry point (fused, twopass, wide, lse) on a GEMM workload whose
    inputs are resident on the GPU; launch() is one forward."""

    def __init__(self, w, variant: str, d):
        import torch
        from gemm_activation_groupnorm_amd import lgn

        self.w, self.variant = w, variant
        dev = "cuda:0"
        self.ws = None
        if variant == "lse":
            self.out = torch.empty(w.M, dtype=torch.float32, device=dev)
            nb = lgn.lgn_lse_workspace_bytes(w.M, w.N)
        else:
            self.out = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
            nb = {"twopass": lgn.lgn_twopass_workspace_bytes(w.M, w.N),
                  "wide": lgn.lgn_wide_workspace_bytes(w.M, w.N)}.get(variant, 0)
        if nb:
            self.ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        out, ws, s = self.out, self.ws, self.stream
        args = (d["x"], d["W"], d["b_lin"], d["b_add"], d["gamma"], d["beta"],
                w.M, w.K, w.N, w.G, w.eps, out)
        f32 = w.dtype == "f32"
        if variant == "fused":
            fn = lgn.lgn_forward_f32 if f32 else lgn.lgn_forward_bf16
            self.launch = lambda: lgn.check(fn(*args, stream=s))
        elif variant == "lse":
            fn = lgn.lgn_linear_lse_f32 if f32 else lgn.lgn_linear_lse_bf16
            largs = (d["x"], d["W"], d["b_lin"], w.M, w.K, w.N, out, ws, nb)
            self.launch = lambda: lgn.check(fn(*largs, stream=s))
        else:
            fn = {("twopass", True): lgn.lgn_forward_twopass_f32,
                  ("twopass", False): lgn.lgn_forward_twopass_bf16,
                  ("wide", True): lgn.lgn_forward_wide_f32,
                  ("wide", False): lgn.lgn_forward_wide_bf16}[(variant, f32)]
            self.launch = lambda: lgn.check(fn(*args, ws, nb, stream=s))

    @property
    def flops(self) -> int:
        return self.w.flops


class SghRunner(_Timed):
    """Swish -> spatial GroupNorm -> HardSwish on y [Nb, C, D*H*W], resident."""

    def __init__(self, w, d):
        import torch
        from gemm_activation_groupnorm_amd import lgn

        self.w, self.variant = w, "sgh"
        self.out = torch.empty_like(d["y"])
        nb = lgn.lgn_sgh_workspace_bytes(w.Nb, w.C, w.S, w.G)
        self.ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda:0")
        self.stream = torch.cuda.current_stream()
        s = self.stream
        args = (d["y"], d["gamma"], d["beta"], w.Nb, w.C, w.S, w.G, w.eps, self.out, self.ws, nb)
        self.launch = lambda: lgn.check(lgn.lgn_swish_gn_hardswish_f32(*args, stream=s))

    @property
    def algorithmic_bytes(self) -> int:
        """One read of y and one write of out (gamma, beta are 2*C floats)."""
        return 2 * self.w.elements * 4 + 2 * self.w.C * 4


class LnConvRunner(_Timed):
    """LayerNorm -> GELU -> dilated Conv1d -> + input on x [B, C, L], resident."""

    def __init__(self, w, d):
        import torch
        from gemm_activation_groupnorm_amd import lgn

        self.w, self.variant = w, "lnconv"
        self.out = torch.empty_like(d["x"])
        nb = lgn.lgn_lnconv_workspace_bytes(w.B, w.C, w.L)
        self.ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda:0")
        self.stream = torch.cuda.current_stream()
        s = self.stream
        args = (d["x"], d["ln_w"], d["ln_b"], d["conv_w"], d["conv_b"], w.B, w.C, w.L, w.dilation,
                w.eps, w.gelu_tanh, self.out, self.ws, nb)
        self.launch = lambda: lgn.check(lgn.lgn_ln_gelu_conv1d_f32(*args, stream=s))

    @property
    def flops(self) -> int:
        return self.w.flops


# ------------------------------------------------------------ workloads ----

class Workload:
    """A workload's seeded inputs (host and device) and its timed entry points."""

    def __init__(self, name: str):
        from gemm_activation_groupnorm_amd import inputs as I
        self.name = name
        t0 = time.perf_counter()
        for lst, kind in ((I.WORKLOADS + I.WIDE_WORKLOADS + I.LSE_WORKLOADS, "gemm"),
                          (I.SGH_WORKLOADS, "sgh"), (I.LNCONV_WORKLOADS, "lnconv")):
            m = [x for x in lst if x.name == name]
            if m:
                self.w, self.kind = m[0], kind
                break
        else:
            raise SystemExit("unknown workload %r" % name)
        w = self.w
        if self.kind == "gemm":
            self.inp = I.workload_inputs(w)
            self.d = gemm_device_inputs(w, self.inp)
            self.dtype = w.dtype
        else:
            import numpy as np
            import torch
            self.inp = (I.make_sgh_inputs(w.Nb, w.C, w.S, w.seed) if self.kind == "sgh" else
                        I.make_lnconv_inputs(w.B, w.C, w.L, w.seed))
            self.d = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0")
                      for k, v in self.inp.items()}
            self.dtype = "f32"
        # hash what the GPU reads (bf16 workloads: the bf16 bits of x and W)
        if self.kind == "gemm" and w.dtype == "bf16":
            hashed = {k: v for k, v in self.inp.items() if k not in ("x", "W")}
        else:
            hashed = self.inp
        self.sha256 = sha256s(hashed)
        eprint("[bench] %s inputs ready in %.1f s" % (name, time.perf_counter() - t0))

    def runner(self, variant: str):
        if self.kind == "sgh":
            return SghRunner(self.w, self.d)
        if self.kind == "lnconv":
            return LnConvRunner(self.w, self.d)
        return Runner(self.w, variant, self.d)

    def release(self):
        import torch
        self.d = None
        torch.cuda.empty_cache()


def measure(wl: Workload, variant: str, steps: int, warmup: int, tel: Telemetry,
            min_warm_ms: float = 0.0, per_launch: bool = False) -> dict:
    """Times one entry point on one workload; returns its record (with the
    output kept on the host for the oracle leg under "_host")."""
    r = wl.runner(variant)
    wall, kmean, t0, t1, w0 = r.time(steps, warmup, min_warm_ms)
    key = "%s/%s" % (wl.name, variant)
    tel.window(key, t0, t1)
    if (tel.summary(key) or {}).get("samples", 0) < MIN_CLOCK_SAMPLES:
        tel.window(key, w0, t1)
    rec = {"workload": wl.name, "variant": variant, "dtype": wl.dtype,
           "ms_per_step": round(wall / steps * 1e3, 4), "kernel_ms_mean": round(kmean, 4),
           "_wall": wall, "_kmean": kmean}
    if wl.kind == "sgh":
        gbps = r.algorithmic_bytes / (kmean * 1e-3) / 1e9
        rec.update(algorithmic_gbps=round(gbps, 1), frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))
        msg = "%.0f GB/s algorithmic (%.1f%% of %.0f)" % (gbps, 100 * gbps / HBM_PEAK_GBPS,
                                                          HBM_PEAK_GBPS)
    else:
        ach = r.flops / (kmean * 1e-3) / 1e12
        peak = PEAK_TFLOPS[wl.dtype]
        rec.update(tflops=round(ach, 3), frac_of_peak=round(ach / peak, 4))
        msg = "%.1f TFLOP/s (%.1f%% of %.1f)" % (ach, 100 * ach / peak, peak)
    if per_launch:
        rec["per_launch"] = r.distributions()
    rec["telemetry"] = tel.summary(key)
    if wl.kind != "sgh":
        rec["frac_of_peak_at_sclk"] = frac_at_clock(rec["tflops"], PEAK_TFLOPS[wl.dtype],
                                                    rec["telemetry"])
    rec["_host"] = r.host_output()
    eprint("[bench] %s: %.3f ms/step, kernel mean %.4f ms -> %s" % (key, wall / steps * 1e3,
                                                                    kmean, msg))
    del r
    return rec


# --------------------------------------------------- cpu_baseline leg ----
# Everything below touches the oracle: its timing on the host, and the
# comparison of every timed output with its fp64 results.

class ErrStats:
    """max abs, mean abs and count above the tolerance over compared elements."""

    def __init__(self, tol: float):
        self.tol, self.max, self.sum, self.n, self.over, self.nonfinite = tol, 0.0, 0.0, 0, 0, 0

    def add(self, y, ref):
        import numpy as np
        fin = np.isfinite(y)
        self.nonfinite += int(y.size - np.count_nonzero(fin))
        d = np.abs(y.astype(np.float64) - ref)
        d[~fin] = np.inf
        if d.size:
            self.max = max(self.max, float(d.max()))
            self.sum += float(d[fin].sum())
        self.n += d.size
        self.over += int(np.count_nonzero(d > self.tol))

    def summary(self) -> dict:
        return {"elements": self.n, "max_abs_err": self.max,
                "mean_abs_err": self.sum / self.n if self.n else 0.0,
                "count_gt_tol": self.over, "nonfinite": self.nonfinite, "tol": self.tol,
                "vs": "fp64 oracle, every element"}


def check_outputs(wl: Workload, recs: list) -> None:
    """Compares every element of each record's output with the oracle (one
    oracle pass per chunk of rows, shared by the workload's records of the
    same method)."""
    lse = [r for r in recs if r["variant"] == "lse"]
    rest = [r for r in recs if r["variant"] != "lse"]
    for group in (lse, rest):
        if group:
            _check_group(wl, group)


def _check_group(wl: Workload, recs: list) -> None:
    import oracle
    t0 = time.perf_counter()
    w, i = wl.w, wl.inp
    if wl.kind == "sgh":
        rows, chunk = w.Nb, 16
        ref_of = lambda a, b: oracle.swish_gn_hardswish(i["y"][a:b], i["gamma"], i["beta"], w.G,
                                                        w.eps)
    elif wl.kind == "lnconv":
        rows, chunk = w.B, 16
        ref_of = lambda a, b: oracle.ln_gelu_conv1d(i["x"][a:b], i["ln_w"], i["ln_b"],
                                                    i["conv_w"], i["conv_b"], w.dilation, w.eps,
                                                    gelu_tanh=w.gelu_tanh)
    elif recs[0]["variant"] == "lse":
        rows, chunk = w.M, 256
        ref_of = lambda a, b: oracle.linear_lse_forward(i["x"][a:b], i["W"], i["b_lin"])
    else:
        rows, chunk = w.M, 2048
        ref_of = lambda a, b: oracle.lgn_forward(i["x"][a:b], i["W"], i["b_lin"], i["b_add"],
                                                 i["gamma"], i["beta"], w.G, w.eps)
    stats = [ErrStats(TOL[wl.dtype]) for _ in recs]
    for a in range(0, rows, chunk):
        b = min(rows, a + chunk)
        ref = ref_of(a, b)
        for st, r in zip(stats, recs):
            st.add(r["_host"][a:b], ref)
    for st, r in zip(stats, recs):
        r["check"] = st.summary()
        eprint("[bench] check %s/%s: max abs %.3e, mean abs %.3e, %d of %d > %.0e (%.1f s)"
               % (wl.name, r["variant"], st.max, r["check"]["mean_abs_err"], st.over, st.n,
                  st.tol, time.perf_counter() - t0))
    if wl.kind == "gemm" and wl.dtype == "bf16" and recs[0]["variant"] != "lse":
        _check_against_unrounded_inputs(wl, recs)


def _check_against_unrounded_inputs(wl: Workload, recs: list) -> None:
    """For information only (the gate is the oracle on the bf16 values the
    GPU reads): the error against the oracle on the fp32 draws before their
    rounding to bf16, i.e. what the bf16 input costs."""
    import oracle
    from gemm_activation_groupnorm_amd import inputs as I
    w = wl.w
    f = I.make_inputs(w.M, w.K, w.N, w.seed, "f32", w.x_scale)
    stats = [ErrStats(TOL["bf16"]) for _ in recs]
    for a in range(0, w.M, 2048):
        b = min(w.M, a + 2048)
        ref = oracle.lgn_forward(f["x"][a:b], f["W"], f["b_lin"], f["b_add"], f["gamma"],
                                 f["beta"], w.G, w.eps)
        for st, r in zip(stats, recs):
            st.add(r["_host"][a:b], ref)
    for st, r in zip(stats, recs):
        info = st.summary()
        info["vs"] = "fp64 oracle on the fp32 inputs before bf16 rounding (information, not a gate)"
        r["check_vs_unrounded_inputs"] = info
        eprint("[bench] %s/%s against the unrounded fp32 inputs: max abs %.3e, mean abs %.3e"
               % (wl.name, r["variant"], st.max, info["mean_abs_err"]))


def cpu_baseline(wl: Workload, variant: str, seconds: float, tmpdir: str) -> dict:
    """The oracle of the headline's method, compiled with -O3 -march=native on
    this host, timed on the first rows (samples) of the workload -- about
    `seconds` of work, OpenMP on every host thread -- and scaled to the
    headline's unit: GEMM (or convolution) TFLOP/s of its fp64 arithmetic, or
    GB/s of the spatial GroupNorm tail's algorithmic bytes."""
    import oracle
    path = oracle.use_native_build(tmpdir)
    w, i = wl.w, wl.inp
    if wl.kind == "sgh":
        total, trial, what = w.Nb, 1, "samples"
        run = lambda n: oracle.swish_gn_hardswish(i["y"][:n], i["gamma"], i["beta"], w.G, w.eps)
        per_unit, unit, scale = 2.0 * w.C * w.S * 4, "GB/s", 1e9
    elif wl.kind == "lnconv":
        total, trial, what = w.B, 1, "samples"
        run = lambda n: oracle.ln_gelu_conv1d(i["x"][:n], i["ln_w"], i["ln_b"], i["conv_w"],
                                              i["conv_b"], w.dilation, w.eps,
                                              gelu_tanh=w.gelu_tanh)
        per_unit, unit, scale = w.flops / w.B, "TFLOP/s", 1e12
    elif variant == "lse":
        total, trial, what = w.M, min(w.M, 16), "rows"
        run = lambda n: oracle.linear_lse_forward(i["x"][:n], i["W"], i["b_lin"])
        per_unit, unit, scale = 2.0 * w.N * w.K, "TFLOP/s", 1e12
    else:
        total, trial, what = w.M, min(w.M, 64), "rows"
        run = lambda n: oracle.lgn_forward(i["x"][:n], i["W"], i["b_lin"], i["b_add"],
                                           i["gamma"], i["beta"], w.G, w.eps)
        per_unit, unit, scale = 2.0 * w.N * w.K, "TFLOP/s", 1e12
    t0 = time.perf_counter()
    run(trial)
    per = (time.perf_counter() - t0) / trial
    n = int(max(trial, min(total, seconds / max(per, 1e-9))))
    t0 = time.perf_counter()
    run(n)
    dt = time.perf_counter() - t0
    hi = host_info()
    return {
        "value": per_unit * n / dt / scale,
        "unit": unit,
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "first %d of %d %s of %s, fp64 C oracle built with %s, %.1f s wall, %d "
                  "OpenMP threads on %s" % (n, total, what, w.name,
                                            " ".join(oracle.NATIVE_CFLAGS[:2]), dt,
                                            oracle.num_threads(), hi["cpu_model"]),
        "cpu_model": hi["cpu_model"],
        "build": os.path.basename(path),
    }


# ----------------------------------------------------------------- main ----

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


# The secondary lines, grouped by workload so that each oracle pass serves
# every entry point timed on it.
EXTRA = [
    (DEFAULT_WORKLOAD, ["fused", "twopass"]),
    ("m32768_k1024_n4096_g64_bf16", ["fused", "twopass"]),
    ("m16384_k2048_n8192_g8_f32", ["fused", "twopass", "wide"]),
    ("m16384_k2048_n8192_g1_f32", ["wide"]),
    ("m1024_k8192_n8192_lse_f32", ["lse"]),
    ("m1024_k8192_n8192_lse_bf16", ["lse"]),
    ("n128_c16_d31_h63_w63_g4_sgh_f32", ["sgh"]),
    ("b32_c256_l4096_d4_lnconv_f32", ["lnconv"]),
]


def headline_workload(workload: str, variant: str) -> str:
    """The workload timed for the headline line: the one asked for, except that a
    variant that cannot run the default fused workload (the other methods, and the
    wide path, whose groups must span 256 channels or more) takes the first
    workload the secondary lines time it on."""
    if variant in ("sgh", "lnconv", "lse", "wide") and workload == DEFAULT_WORKLOAD:
        return [n for n, v in EXTRA if variant in v][0]
    return workload


METHOD_NAMES = {
    "fused": "fused Linear+Swish+bias+GroupNorm",
    "twopass": "two-pass Linear+Swish+bias+GroupNorm (GEMM, then the GroupNorm epilogue kernel)",
    "wide": "wide-group Linear+Swish+bias+GroupNorm (fused tile, then the normalise kernel)",
    "lse": "Linear->logsumexp->LeakyReLU x2->GELU x2",
}


def fused_runs_two_kernels(w) -> bool:
    """The fused entry points' own dispatch (include/lgn.h): fp32 inputs with
    512 or more channels per group and K a positive multiple of 16, or bf16
    inputs with 1024 channels per group and K >= 2048 a multiple of 32, run
    the GEMM and the GroupNorm epilogue as two kernels."""
    c = w.N // w.G
    if w.dtype == "f32":
        return c >= 512 and w.K >= 16 and w.K % 16 == 0
    return c == 1024 and w.K >= 2048 and w.K % 32 == 0


def gemm_metric(w, variant: str) -> str:
    """The headline metric's name for a GEMM-family line: the contract's own
    name for the fused forward at 32768 x 1024 x 4096, else the method and
    the shape it was measured on."""
    if variant == "fused" and (w.M, w.K, w.N) == (32768, 1024, 4096):
        return METRIC
    shape = "M%d K%d N%d" % (w.M, w.K, w.N) + ("" if variant == "lse" else " G%d" % w.G)
    return "%s TFLOP/s at %s %s; %% MFMA peak" % (METHOD_NAMES[variant], shape, w.dtype)


def headline_json(wl: Workload, rec: dict, args) -> dict:
    w = wl.w
    wall, kmean = rec["_wall"], rec["_kmean"]
    ms = wall / args.steps * 1e3
    base = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": wl.dtype, "data": "synthetic"}
    cfg = {"workload": w.name, "variant": rec["variant"], "seed": w.seed, "eps": w.eps,
           "inputs_sha256": wl.sha256}
    if wl.kind == "sgh":
        gbps = rec["algorithmic_gbps"]
        cfg.update(Nb=w.Nb, C=w.C, D=w.D, H=w.H, W=w.W, G=w.G)
        return {"metric": "Swish->spatial GroupNorm->HardSwish algorithmic HBM GB/s",
                "value": round((2 * w.elements * 4 + 2 * w.C * 4) / (ms * 1e-3) / 1e9, 1),
                "unit": "GB/s", **base, "config": cfg,
                "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                             "traffic": traffic_for(w.name, "sgh"),
                             "kernel_ms_mean": round(kmean, 4),
                             "kernel": "lgn_sgh_clear_kernel+lgn_sgh_onepass_kernel"}}
    ach = w.flops / (kmean * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    if wl.kind == "lnconv":
        cfg.update(B=w.B, C=w.C, L=w.L, dilation=w.dilation,
                   gelu="tanh" if w.gelu_tanh else "exact")
        metric = "LayerNorm->GELU->dilated Conv1d->+x convolution TFLOP/s"
        kernel = "wpack+stats+lnconv"
    else:
        cfg.update(M=w.M, K=w.K, N=w.N, G=w.G,
                   inputs="x~%g*N(0,1); W,b_lin~U(+-1/sqrt(K)); b_add~0.02*N(0,1); "
                          "gamma~1+0.1*N(0,1); beta~0.1*N(0,1)" % w.x_scale)
        metric = gemm_metric(w, rec["variant"])
        kernel = {"fused": "lgn_fused_kernel", "twopass": "gemm+epilogue",
                  "wide": "wide partial+norm", "lse": "lse partial+finish"}[rec["variant"]]
        if rec["variant"] == "fused" and fused_runs_two_kernels(w):
            kernel = "gemm+epilogue (fused entry point at %d channels per group)" % (w.N // w.G)
    return {"metric": metric, "value": round(w.flops / (ms * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s", **base, "config": cfg,
            "roofline": {"bound": "mfma", "achieved": round(ach, 3), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                         "traffic": traffic_for(w.name, rec["variant"]),
                         "kernel_ms_mean": round(kmean, 4), "kernel": kernel,
                         "frac_at_sclk": frac_at_clock(ach, peak, rec.get("telemetry"))}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", default="fused",
                    choices=["fused", "twopass", "wide", "lse", "sgh", "lnconv"],
                    help="lse: Linear -> logsumexp -> LeakyReLU x2 -> GELU x2; sgh: Swish -> "
                         "spatial GroupNorm -> HardSwish (reports GB/s); lnconv: LayerNorm -> "
                         "GELU -> dilated Conv1d -> + x.  Without --workload these three take "
                         "their own default workload (m1024_k8192_n8192_lse_f32, "
                         "n128_c16_d31_h63_w63_g4_sgh_f32, b32_c256_l4096_d4_lnconv_f32)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg: no CPU baseline and no per-line check")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads and entry points")
    ap.add_argument("--no-per-launch", action="store_true",
                    help="skip the per-launch (median/p10/p90, flushed) timings, e.g. under a "
                         "profiler whose kernel averages should cover the timed launches only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--torch-context", action="store_true",
                    help="also time, for context only, torch's linear (vendor GEMM) and the "
                         "unfused torch pipeline on the same workload")
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

    tel = Telemetry().start()
    head_name, head_var = headline_workload(args.workload, args.variant), args.variant
    groups = [(head_name, [head_var])]
    if not args.no_extra:
        for name, variants in EXTRA:
            vs = [v for v in variants if not (name == head_name and v == head_var)]
            if name == head_name:
                groups[0][1].extend(vs)
            elif vs:
                groups.append((name, vs))

    # The headline's group is timed last, after the other workloads: on a GPU
    # that was idle the sysfs clock reading trails the real clock for a few
    # hundred milliseconds, and the headline's telemetry would read that lag.
    # Its own W warm-up launches and K timed ones are unchanged.
    head_rec, head_wl, extra, measured = None, None, [], []
    for gi in list(range(1, len(groups))) + [0]:
        name, variants = groups[gi]
        wl = Workload(name)
        if gi == 0:
            head_wl = wl
        recs = []
        for v in variants:
            if gi == 0 and v == head_var:
                rec = measure(wl, v, args.steps, args.warmup, tel,
                              per_launch=not args.no_per_launch)
                head_rec = rec
            else:
                per = (not args.no_per_launch) and v == "fused" and wl.dtype == "bf16"
                rec = measure(wl, v, 50, 5, tel, min_warm_ms=100.0, per_launch=per)
                extra.append(rec)
            recs.append(rec)
        wl.release()
        measured.append((wl, recs))
    tel.stop()

    res = headline_json(head_wl, head_rec, args)
    if head_rec.get("per_launch"):
        res["per_launch"] = head_rec["per_launch"]
    res["telemetry"] = {"gpu": head_rec["telemetry"], "gpu_source": tel.source,
                        "host": host_info()}
    if args.torch_context:
        res["torch_context"] = torch_context(head_wl.w)

    res["check"] = None
    res["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        for wl, recs in measured:
            check_outputs(wl, recs)
        res["check"] = head_rec["check"]
        if "check_vs_unrounded_inputs" in head_rec:
            res["check_vs_unrounded_inputs"] = head_rec["check_vs_unrounded_inputs"]
        with tempfile.TemporaryDirectory() as td:
            res["cpu_baseline"] = cpu_baseline(head_wl, head_rec["variant"], args.cpu_seconds, td)
            eprint("[bench] cpu baseline: %s" % res["cpu_baseline"]["sample"])
    for r in extra:
        for k in [k for k in r if k.startswith("_")]:
            del r[k]
    if extra:
        res["extra"] = extra
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
