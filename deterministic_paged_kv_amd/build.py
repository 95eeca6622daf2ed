"""Compile the HIP libraries in-tree for gfx950 (hipcc; no GPU needed to build): libpa.so (the
attention library of include/pa.h) and libpa_probe.so (the measurement kernels of
include/pa_probe.h that the benchmark reports ceilings with)."""

from __future__ import annotations

import concurrent.futures
import os
import re
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


# Resource-usage remarks of a compile: every kernel must use no scratch.  Several kernels wait
# for their direct-to-LDS loads with hand-counted vmcnt values, and a register spill inside
# such a loop would add memory operations to that count (and make the waits wrong), so a
# spilling build is an error rather than a slow kernel.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
_NAME = re.compile(r"remark:\s+Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def check_no_scratch(source: str, remarks: str) -> None:
    name = None
    for line in remarks.splitlines():
        m = _NAME.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) != 0:
            raise RuntimeError(f"{source}: kernel {name} uses {m.group(1)} bytes of scratch per lane")


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libpa.so and libpa_probe.so next to this file; returns the
    path of libpa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    objs = {s: os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs}
    cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, []), *RESOURCE_REMARKS, "-c", os.path.join(CSRC, s), "-o", objs[s]]
            for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for src, r in zip(srcs, ex.map(_run, cmds)):
            check_no_scratch(src, r.stderr)
            if verbose:
                sys.stderr.write("".join(l + "\n" for l in r.stderr.splitlines() if "remark" not in l and l.strip()
                                         and not l.lstrip()[:1].isdigit() and "|" not in l))
    for lib, names in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[objs[s] for s in names], "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
