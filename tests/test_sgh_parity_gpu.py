"""GPU parity of Swish -> spatial GroupNorm -> HardSwish (through the C ABI)
against the fp64 oracle; max abs error <= 2e-4 (fp32 data)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import SGH_WORKLOADS, make_sgh_inputs
from gpu_helpers import TOL, compare_all_rows, log

pytestmark = pytest.mark.gpu


def run_sgh(d, Nb, C, S, G, eps, out=None, stream=None):
    if out is None:
        out = torch.empty((Nb, C, S), dtype=torch.float32, device="cuda")
    nb = lgn.lgn_sgh_workspace_bytes(Nb, C, S, G)
    ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
    lgn.check(lgn.lgn_swish_gn_hardswish_f32(d["y"], d["gamma"], d["beta"], Nb, C, S, G, eps, out,
                                             ws, nb, stream=stream))
    return out


def dev(inp):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}


def _err(y, ref):
    assert np.all(np.isfinite(y)), "non-finite GPU output"
    return float(np.max(np.abs(y.astype(np.float64) - ref))) if y.size else 0.0


SHAPES = [
    # Nb, C, S, G
    (2, 16, 123039 // 37, 4),   # odd S: group slabs start off 16-byte boundaries
    (1, 4, 1, 4),               # one element per group
    (3, 8, 100, 2),             # S < one wave's stride
    (2, 6, 5000, 3),            # several chunks per group, ragged last chunk
    (1, 2, 16384 * 2, 1),       # exactly two full chunks
    (4, 16, 777, 16),           # one channel per group (instance-norm shape)
    (2, 12, 4099, 1),           # one group over all channels
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "Nb%d_C%d_S%d_G%d" % s)
def test_sgh_shapes(shape):
    Nb, C, S, G = shape
    log("sgh case Nb=%d C=%d S=%d G=%d" % shape)
    inp = make_sgh_inputs(Nb, C, S, 700 + Nb + C + S + G)
    out = run_sgh(dev(inp), Nb, C, S, G, 1e-5)
    torch.cuda.synchronize()
    ref = oracle.swish_gn_hardswish(inp["y"], inp["gamma"], inp["beta"], G, 1e-5)
    err = _err(out.cpu().numpy(), ref)
    log("  max abs err %.3e" % err)
    assert err <= TOL["f32"]


def test_sgh_in_place_and_deterministic():
    Nb, C, S, G = 2, 8, 20000, 4
    inp = make_sgh_inputs(Nb, C, S, 71)
    d = dev(inp)
    a = run_sgh(d, Nb, C, S, G, 1e-5)
    b = run_sgh(d, Nb, C, S, G, 1e-5)
    buf = d["y"].clone()
    run_sgh(dict(d, y=buf), Nb, C, S, G, 1e-5, out=buf)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "run-to-run difference"
    assert torch.equal(a, buf), "in place differs"


def test_sgh_constant_group_gives_hardswish_beta():
    # zero variance: eps alone scales the (fp32-rounded) deviations by
    # 1/sqrt(eps) ~ 316, so the bar is the parity tolerance, not exactness
    Nb, C, S, G = 1, 4, 3000, 2
    inp = make_sgh_inputs(Nb, C, S, 72)
    inp["y"][0, 2:4] = np.float32(0.7)
    out = run_sgh(dev(inp), Nb, C, S, G, 1e-5).cpu().numpy()
    ref = oracle.hardswish(inp["beta"][2:4].astype(np.float64))
    assert np.max(np.abs(out[0, 2:4] - ref[:, None])) <= TOL["f32"]
    full = oracle.swish_gn_hardswish(inp["y"], inp["gamma"], inp["beta"], G, 1e-5)
    assert _err(out, full) <= TOL["f32"]


@pytest.mark.parametrize("wi", range(len(SGH_WORKLOADS)))
def test_sgh_full_size_every_element(wi):
    w = SGH_WORKLOADS[wi]
    log("sgh workload %s" % w.name)
    inp = make_sgh_inputs(w.Nb, w.C, w.S, w.seed)
    out = run_sgh(dev(inp), w.Nb, w.C, w.S, w.G, w.eps)
    torch.cuda.synchronize()
    host = out.cpu().numpy()
    del out
    # whole samples at a time (their groups are complete), every element
    stats = compare_all_rows(
        {"sgh": host},
        lambda r0, r1: oracle.swish_gn_hardswish(inp["y"][r0:r1], inp["gamma"], inp["beta"],
                                                 w.G, w.eps),
        w.Nb, TOL["f32"], chunk=16)
    log("  every element: %s" % stats["sgh"])
    assert stats["sgh"].n == w.elements and stats["sgh"].max <= TOL["f32"]


# Chunks with no whole 16-byte float4 inside them: a group whose length
# leaves 5 or 6 elements in its last chunk, starting 1 or 2 elements past a
# 16-byte boundary, must still cover every element exactly once (head and
# tail of up to 3 each).
EDGE_SHAPES = [
    (1, 2, 5, 2),        # groups of 5 elements starting at 0 and 5
    (2, 4, 5, 4),        # 8 groups of 5: starts 0, 5, 10, ... cover every residue mod 4
    (2, 16, 16389, 16),  # last chunk of each group holds 5 elements
    (3, 6, 16390, 3),    # last chunk of 6 elements, groups of 2 channels
    (1, 3, 7, 3),        # groups of 7 starting at 0, 7, 14
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "Nb%d_C%d_S%d_G%d" % s)
def test_sgh_chunks_without_a_whole_float4(shape):
    Nb, C, S, G = shape
    log("sgh edge case Nb=%d C=%d S=%d G=%d" % shape)
    inp = make_sgh_inputs(Nb, C, S, 800 + Nb + C + S + G)
    d = dev(inp)
    # the output starts as NaN: an element the kernels skip stays NaN and fails
    out = torch.full((Nb, C, S), float("nan"), dtype=torch.float32, device="cuda")
    run_sgh(d, Nb, C, S, G, 1e-5, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "elements left unwritten"
    ref = oracle.swish_gn_hardswish(inp["y"], inp["gamma"], inp["beta"], G, 1e-5)
    err = _err(got, ref)
    log("  max abs err %.3e" % err)
    assert err <= TOL["f32"]


# ---- the single-pass form against the two-kernel form ----
#
# Out of place (and at most 256 chunks per group) the call runs one kernel
# that reads y once; in place it runs the statistics and apply kernels.
# Both must give bitwise the same output, and so must the single-pass
# kernel's own fallback (statistics formed from y when its bounded wait for
# the rest of the group runs out), forced here with a wait of zero polls.

ONEPASS_SHAPES = [
    (2, 16, 123039 // 37, 4),    # odd S, groups off 16-byte boundaries
    (3, 6, 16390, 3),            # a 6-element last chunk per group
    (4, 16, 777, 16),            # one channel per group
    (1, 8, 16384 * 9 + 3, 2),    # 37 chunks per group
    (2, 2048, 5, 2),             # 1024 channels per group (the 1024 coefficient table)
    (1, 16384, 2, 2),            # 8192 channels per group (the 8192 coefficient table)
    (1, 1, 16384 * 256, 1),      # 256 chunks per group: the single pass's limit
    (1, 2, 16384 * 128 - 1, 1),  # 256 chunks, the last one 16382 elements
]


@pytest.mark.parametrize("shape", ONEPASS_SHAPES, ids=lambda s: "Nb%d_C%d_S%d_G%d" % s)
def test_sgh_single_pass_equals_two_kernels_and_its_fallback(shape):
    Nb, C, S, G = shape
    log("sgh single pass vs two kernels Nb=%d C=%d S=%d G=%d" % shape)
    inp = make_sgh_inputs(Nb, C, S, 900 + Nb + C + S + G)
    d = dev(inp)
    one = run_sgh(d, Nb, C, S, G, 1e-5)                      # out of place: single pass
    buf = d["y"].clone()
    run_sgh(dict(d, y=buf), Nb, C, S, G, 1e-5, out=buf)      # in place: two kernels
    try:
        lgn.lgn_testing_set_sgh_spin_limit(0)
        fb = run_sgh(d, Nb, C, S, G, 1e-5)                   # single pass, fallback route
        torch.cuda.synchronize()
    finally:
        lgn.lgn_testing_set_sgh_spin_limit(-1)
    assert torch.equal(one, buf), "single pass differs from the two-kernel path"
    assert torch.equal(one, fb), "single pass differs from its fallback route"
    ref = oracle.swish_gn_hardswish(inp["y"], inp["gamma"], inp["beta"], G, 1e-5)
    err = _err(one.cpu().numpy(), ref)
    log("  bitwise equal on all three routes; max abs err %.3e" % err)
    assert err <= TOL["f32"]


def test_sgh_groups_beyond_the_single_pass_take_two_kernels():
    # 257 chunks per group: over the single-pass limit, the two-kernel path
    Nb, C, S, G = 1, 1, 16384 * 256 + 7, 1
    log("sgh 257-chunk group")
    inp = make_sgh_inputs(Nb, C, S, 41)
    out = run_sgh(dev(inp), Nb, C, S, G, 1e-5)
    torch.cuda.synchronize()
    ref = oracle.swish_gn_hardswish(inp["y"], inp["gamma"], inp["beta"], G, 1e-5)
    err = _err(out.cpu().numpy(), ref)
    log("  max abs err %.3e" % err)
    assert err <= TOL["f32"]


def test_sgh_single_pass_calls_overlapping_on_two_streams():
    # Two single-pass calls in flight at once, each with its own workspace.
    # They share the GPU, so a group's chunks need not all be resident at the
    # same time; a wait that runs out falls back to forming the statistics
    # from y.  Either way each output must be bitwise that of the same call
    # made alone.
    shapes = [(8, 16, 31 * 63 * 9, 4), (6, 8, 16384 * 20 + 5, 2)]
    calls = []
    for k, (Nb, C, S, G) in enumerate(shapes):
        inp = make_sgh_inputs(Nb, C, S, 950 + k)
        d = dev(inp)
        nb = lgn.lgn_sgh_workspace_bytes(Nb, C, S, G)
        ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
        alone = torch.empty((Nb, C, S), dtype=torch.float32, device="cuda")
        both = torch.full((Nb, C, S), float("nan"), dtype=torch.float32, device="cuda")
        calls.append((d, Nb, C, S, G, nb, ws, alone, both))
    log("sgh single pass alone, then two streams at once: %s" % (shapes,))
    for d, Nb, C, S, G, nb, ws, alone, both in calls:
        lgn.check(lgn.lgn_swish_gn_hardswish_f32(d["y"], d["gamma"], d["beta"], Nb, C, S, G,
                                                 1e-5, alone, ws, nb))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for st, (d, Nb, C, S, G, nb, ws, alone, both) in zip(streams, calls):
            lgn.check(lgn.lgn_swish_gn_hardswish_f32(d["y"], d["gamma"], d["beta"], Nb, C, S, G,
                                                     1e-5, both, ws, nb, stream=st))
    torch.cuda.synchronize()
    for d, Nb, C, S, G, nb, ws, alone, both in calls:
        assert torch.equal(alone, both)
