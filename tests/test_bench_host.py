"""bench.py's host-side pieces without a GPU: the error statistics of its
check leg, the input hashes, the host description, the CPU-baseline leg of
every headline variant and the refusal of multi-GPU runs."""
import hashlib
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_err_stats_counts_every_element():
    st = bench.ErrStats(1e-3)
    ref = np.zeros((3, 4))
    y = np.zeros((3, 4), dtype=np.float32)
    y[0, 0] = 2e-3
    y[2, 3] = -5e-4
    st.add(y[:2], ref[:2])
    st.add(y[2:], ref[2:])
    s = st.summary()
    assert s["elements"] == 12 and s["count_gt_tol"] == 1 and s["nonfinite"] == 0
    assert abs(s["max_abs_err"] - 2e-3) < 1e-9
    assert abs(s["mean_abs_err"] - (2e-3 + 5e-4) / 12) < 1e-9


def test_err_stats_flags_non_finite_output():
    st = bench.ErrStats(1e-3)
    y = np.array([0.0, np.nan, np.inf], dtype=np.float32)
    st.add(y, np.zeros(3))
    s = st.summary()
    assert s["nonfinite"] == 2 and s["count_gt_tol"] == 2 and s["max_abs_err"] == np.inf


def test_input_hashes_are_sha256_of_the_bytes():
    a = np.arange(10, dtype=np.float32)
    h = bench.sha256s({"a": a})
    assert h["a"] == hashlib.sha256(a.tobytes()).hexdigest()


def test_host_info_names_the_cpu():
    hi = bench.host_info()
    assert hi["logical_cpus"] == os.cpu_count() and hi["usable_cpus"] >= 1
    assert hi["cpu_model"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def _fake(kind, w, inp):
    """A stand-in for bench.Workload: its host inputs and shape, no device."""
    import types
    return types.SimpleNamespace(kind=kind, w=w, inp=inp, name=w.name)


def _baseline_cases():
    from gemm_activation_groupnorm_amd import inputs as I
    gw = I.Workload("tiny_f32", 64, 32, 128, 8, "f32", 0)
    sw = I.SghWorkload("tiny_sgh", 3, 8, 2, 3, 5, 2, 7)
    cw = I.LnConvWorkload("tiny_lnconv", 2, 8, 16, 2, 9)
    return [
        ("gemm", "fused", gw, I.workload_inputs(gw), "TFLOP/s", "rows"),
        ("gemm", "lse", gw, I.workload_inputs(gw), "TFLOP/s", "rows"),
        ("sgh", "sgh", sw, I.make_sgh_inputs(sw.Nb, sw.C, sw.S, sw.seed), "GB/s", "samples"),
        ("lnconv", "lnconv", cw, I.make_lnconv_inputs(cw.B, cw.C, cw.L, cw.seed), "TFLOP/s",
         "samples"),
    ]


def test_cpu_baseline_covers_every_headline_variant(tmp_path):
    import oracle
    try:
        for kind, variant, w, inp, unit, what in _baseline_cases():
            cb = bench.cpu_baseline(_fake(kind, w, inp), variant, 0.05, str(tmp_path))
            assert cb["unit"] == unit and cb["kind"] == "oracle", (variant, cb)
            assert cb["value"] > 0 and cb["cores"] >= 1
            assert (" %s of %s," % (what, w.name)) in cb["sample"]
    finally:
        oracle.use_default_build()


def test_fraction_at_the_measured_clock():
    tel = {"samples": 12, "sclk_mhz": {"min": 1800.0, "median": 1800.0, "max": 1800.0}}
    # 900 of a 2500 peak quoted at 2400 MHz: at 1800 MHz the peak is 1875
    assert bench.frac_at_clock(900.0, 2500.0, tel) == 0.48
    # too few readings to stand for the region
    assert bench.frac_at_clock(900.0, 2500.0, dict(tel, samples=2)) is None
    # readings still ramping up from idle
    ramp = {"samples": 9, "sclk_mhz": {"min": 1053.0, "median": 1516.0, "max": 1820.0}}
    assert bench.frac_at_clock(140.0, 157.3, ramp) is None
    assert bench.frac_at_clock(900.0, 2500.0, {"samples": 0}) is None
    assert bench.frac_at_clock(900.0, 2500.0, None) is None


def test_check_leg_splits_methods_sharing_a_workload(monkeypatch):
    """A workload timed with both the GroupNorm forward and the logsumexp
    method: each record is compared with its own method's oracle."""
    import types
    from gemm_activation_groupnorm_amd import inputs as I
    import oracle
    w = I.Workload("tiny_f32", 64, 32, 128, 8, "f32", 0)
    inp = I.workload_inputs(w)
    wl = types.SimpleNamespace(kind="gemm", w=w, inp=inp, name=w.name, dtype="f32")
    fwd = oracle.lgn_forward(inp["x"], inp["W"], inp["b_lin"], inp["b_add"], inp["gamma"],
                             inp["beta"], w.G, w.eps).astype(np.float32)
    lse = oracle.linear_lse_forward(inp["x"], inp["W"], inp["b_lin"]).astype(np.float32)
    recs = [{"variant": "lse", "_host": lse}, {"variant": "fused", "_host": fwd},
            {"variant": "twopass", "_host": fwd}]
    bench.check_outputs(wl, recs)
    for r in recs:
        assert r["check"]["count_gt_tol"] == 0 and r["check"]["elements"] == r["_host"].size


def test_metric_names_the_method_and_shape():
    from gemm_activation_groupnorm_amd import inputs as I
    head = I.get_workload("m32768_k1024_n4096_g64_f32")
    assert bench.gemm_metric(head, "fused") == bench.METRIC
    lse = [w for w in I.LSE_WORKLOADS if w.dtype == "f32"][0]
    m = bench.gemm_metric(lse, "lse")
    assert m.startswith("Linear->logsumexp") and "M1024 K8192 N8192" in m
    assert "two-pass" in bench.gemm_metric(head, "twopass")


def test_bf16_lines_also_report_the_unrounded_input_error():
    """The bf16 gate is the oracle on the bf16 values; the error against the
    fp32 draws before rounding is reported beside it as information."""
    import types
    from gemm_activation_groupnorm_amd import inputs as I
    import oracle
    w = I.Workload("tiny_bf16", 64, 32, 128, 8, "bf16", 3)
    inp = I.workload_inputs(w)
    wl = types.SimpleNamespace(kind="gemm", w=w, inp=inp, name=w.name, dtype="bf16")
    y = oracle.lgn_forward(inp["x"], inp["W"], inp["b_lin"], inp["b_add"], inp["gamma"],
                           inp["beta"], w.G, w.eps).astype(np.float32)
    recs = [{"variant": "fused", "_host": y}]
    bench.check_outputs(wl, recs)
    r = recs[0]
    assert r["check"]["max_abs_err"] < 1e-5          # exact oracle on the bf16 values
    info = r["check_vs_unrounded_inputs"]
    assert "not a gate" in info["vs"] and info["elements"] == y.size
    assert info["max_abs_err"] > r["check"]["max_abs_err"]   # the rounding shows


def test_headline_workload_defaults_per_variant():
    import bench
    d = bench.DEFAULT_WORKLOAD
    assert bench.headline_workload(d, "fused") == d
    assert bench.headline_workload(d, "twopass") == d
    assert bench.headline_workload(d, "wide") == "m16384_k2048_n8192_g8_f32"
    assert bench.headline_workload(d, "lse") == "m1024_k8192_n8192_lse_f32"
    assert bench.headline_workload(d, "sgh") == "n128_c16_d31_h63_w63_g4_sgh_f32"
    assert bench.headline_workload(d, "lnconv") == "b32_c256_l4096_d4_lnconv_f32"
    # an explicit workload is kept
    assert bench.headline_workload("m16384_k2048_n8192_g1_f32", "wide") == "m16384_k2048_n8192_g1_f32"
