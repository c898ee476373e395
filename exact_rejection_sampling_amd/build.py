"""Builds libspec_verify.so (hand-written HIP kernels for gfx950 + the C ABI) in-tree.

    python -m exact_rejection_sampling_amd.build

Each source is compiled with hipcc for gfx950 only, then linked into
exact_rejection_sampling_amd/libspec_verify.so.  Object files go to _build/ at the
repository root.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspec_verify.so")
SOURCES = ["abi.hip", "chain.hip", "greedy.hip", "tree.hip", "proc.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # packed fp32 instructions stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand) and shutil.which(cand) is None:
        raise RuntimeError("hipcc not found: set HIPCC or install ROCm")
    return cand


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


TRACE_LIB = os.path.join(PKG, "libspec_verify_trace.so")


def build_library(verbose: bool = False, jobs: int = 4, trace: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path.

    trace=True builds the timeline-trace variant instead (-DSPEC_TRACE, objects under
    _build/trace, library libspec_verify_trace.so): the same kernels with per-block
    real-time stamps, for profiling only (spec_trace_set in include/spec_verify.h)."""
    cc = hipcc()
    build = os.path.join(BUILD, "trace") if trace else BUILD
    lib = TRACE_LIB if trace else LIB
    extra = ["-DSPEC_TRACE=1"] if trace else []
    os.makedirs(build, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv, trace="--trace" in sys.argv))
