"""Builds libbitlinear.so (gfx950) in-tree with hipcc.

Usage: ``python -m w1_a8_matmul_amd.build`` or ``build_library()``.
Objects go to ``_build/`` at the repository root; the library lands next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libbitlinear.so")
# Measurement-only probes (streaming read, int8 matrix-core loop) for bench.py.
PROBES_LIBRARY = os.path.join(PKG, "libbitlinear_probes.so")
PROBES_SOURCES = ["probes.hip"]

SOURCES = ["abi.cpp", "weights.hip", "acts.hip", "gemv.hip", "gemm.hip", "group.hip",
           "lut.hip", "chain.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: the float epilogue must be two separate IEEE roundings.
# Correctly rounded fp32 division is HIP's default; it is spelled out here
# because the quantizers depend on it.  Packed fp32 instructions are kept off.
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-Wno-inline-asm",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if l.strip() and noise not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs, target: str) -> None:
    tmp = target + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, target)


def build_library(jobs: int = 8) -> str:
    """Builds libbitlinear.so and the probe library; returns the former's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBES_SOURCES
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIBRARY)
    _link(objs[len(SOURCES):], PROBES_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_library())
