"""Compile the HIP libraries in-tree for gfx950 (hipcc; no GPU needed to build): libpa.so (the
attention library of include/pa.h) and libpa_probe.so (the measurement kernels of
include/pa_probe.h that the benchmark reports ceilings with)."""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_api.hip", "pa_validate.hip", "pa_decode.hip", "pa_prefill.hip", "pa_csr.hip", "pa_backward.hip"]
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
PROBE_SOURCES = ["pa_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed FP32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# MFMA accumulators in ordinary VGPRs: the kernels rescale them on the VALU
EXTRA = {
    "pa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "pa_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "pa_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libpa.so and libpa_probe.so next to this file; returns the
    path of libpa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    objs = {s: os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs}
    cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", objs[s]] for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for r in ex.map(_run, cmds):
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    for lib, names in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[objs[s] for s in names], "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
