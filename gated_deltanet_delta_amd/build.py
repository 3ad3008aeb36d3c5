"""Build libgdn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m gated_deltanet_delta_amd.build        # or: from ... import build; build.build()

Objects go to <repo>/_build/, the library to gated_deltanet_delta_amd/libgdn.so.
Beside it, libgdn_debug.so: the same kernels with the C ABI built with
GDN_DEBUG_CHECKS (each call also checks on the device that its slot ids are
distinct, GDN_DEV_DUP_SLOT).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
LIB_DEBUG = os.path.join(PKG, "libgdn_debug.so")

HIP_SOURCES = ["gdn_step.hip", "gdn_prefill.hip"]
HOST_SOURCES = ["gdn_api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # MFMA accumulators in VGPRs: the chained products feed them straight to VALU
    # code and the next MFMA, so AGPR<->VGPR copies would only add instructions
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libgdn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    incs = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj])
    debug_objs = list(objs)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        dobj = os.path.join(BUILD, src + ".debug.o")
        objs.append(obj)
        debug_objs.append(dobj)
        jobs.append(["g++", *HOST_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj])
        jobs.append(["g++", *HOST_FLAGS, "-DGDN_DEBUG_CHECKS=1", *incs, "-c", os.path.join(CSRC, src), "-o", dobj])
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    for lib, lib_objs in ((LIB, objs), (LIB_DEBUG, debug_objs)):
        tmp = lib + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *lib_objs], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
