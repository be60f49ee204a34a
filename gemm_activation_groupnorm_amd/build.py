"""Builds liblgn.so (the HIP library behind include/lgn.h) in-tree for gfx950.

    python -m gemm_activation_groupnorm_amd.build

Every .hip file in csrc/ is compiled to an object under _build/ (in
parallel), then linked into gemm_activation_groupnorm_amd/liblgn.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "lgn")
LIB = os.path.join(PKG, "liblgn.so")
# Stand-alone measurement probe (not part of the library): the sustained MFMA
# rate and shader clock for zero and random operands.
PROBE_SRC = os.path.join(PKG, "probes", "mfma_ceiling.hip")
PROBE = os.path.join(PKG, "probes", "mfma_ceiling")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    # the host pass does not know the gfx950 feature named above; that warning is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if warn:
        sys.stderr.write(warn + "\n")
    return obj


def build(jobs: int = 8, extra=()) -> str:
    """Compile every csrc/*.hip and link liblgn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> str:
    """Compile the MFMA-ceiling probe executable next to its source."""
    tmp = PROBE + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), *[f for f in HIPCC_FLAGS if f != "-fPIC"], PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SRC, " ".join(cmd), r.stderr))
    os.replace(tmp, PROBE)
    return PROBE


if __name__ == "__main__":
    print(build())
