"""Compile the HIP library libpa.so in-tree for gfx950 (hipcc; no GPU needed to build)."""

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
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libpa.so next to this file; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for r in ex.map(_run, cmds):
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
