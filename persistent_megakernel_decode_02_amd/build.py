"""Build libmkd.so (HIP for gfx950 + host C++) in-tree.

Usage: ``python -m persistent_megakernel_decode_02_amd.build`` (always
recompiles).  Objects go to ``_build/`` at the repository root; the shared
library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmkd.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed fp32 ops are disabled for all device code: the compiler otherwise
# forms v_pk_* fp32 instructions from ordinary float code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I" + INCLUDE, "-I" + CSRC]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-I" + os.path.join(ROCM, "include")]


def _run(cmd):
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return time.time() - t


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    steps = [
        ([HIPCC] + DEVICE_FLAGS + ["-c", os.path.join(CSRC, "mkd_kernel.hip")], "mkd_kernel.o"),
        ([HIPCC] + HOST_FLAGS + ["-D__HIP_PLATFORM_AMD__", "-x", "c++", "-c",
                                 os.path.join(CSRC, "mkd_api.cpp")], "mkd_api.o"),
        (["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, "schedule.cpp")], "schedule.o"),
    ]
    for cmd, obj in steps:
        out = os.path.join(BUILD, obj)
        dt = _run(cmd + ["-o", out])
        objs.append(out)
        if verbose:
            print(f"[build] {obj} ({dt:.1f}s)", flush=True)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build()
