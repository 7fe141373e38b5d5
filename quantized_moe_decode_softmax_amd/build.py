"""Builds libmoe.so (HIP kernels for gfx950 + host code) in the package directory.

    python -m quantized_moe_decode_softmax_amd.build

The host-only part (validation, layout, packing) is compiled with g++; the HIP
sources with hipcc for gfx950 only. Packed FP32 instructions are disabled
(-packed-fp32-ops): the kernels are written for scalar/dual-issue fp32.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
TRACE_LIB = os.path.join(PKG, "libmoe_trace.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["gen.hip", "decode.hip", "stack1.hip", "noalloc.hip", "dense.hip", "attention.hip", "gdn.hip"]
HOST_SOURCES = ["moe_host.cpp"]
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, phase_trace: bool = False) -> str:
    """Builds libmoe.so; phase_trace=True builds libmoe_trace.so instead, whose
    streaming stack kernel also writes per-phase timestamps into the workspace
    (compiled with MOE_PHASE_TRACE; a measurement build, never the product)."""
    bdir = BUILD + ("_trace" if phase_trace else "")
    lib = TRACE_LIB if phase_trace else LIB
    defs = ["-DMOE_PHASE_TRACE=1"] if phase_trace else []
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        jobs.append(["g++", "-O2", "-fPIC", "-std=c++17", "-Wall", *defs, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        jobs.append([HIPCC, *HIP_FLAGS, *defs, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_trace="--phase-trace" in sys.argv))
