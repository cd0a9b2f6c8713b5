"""Build libmkd.so (HIP for gfx950 + host C++) in-tree.

Usage: ``python -m persistent_megakernel_decode_02_amd.build`` (recompiles
everything; ``--incremental`` only what changed).  Objects go to ``_build/`` at the repository root; the shared
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


# device translation units (each kernel on its own, so they compile in
# parallel) and host ones; every object depends on the headers too
DEVICE_SRCS = ["mkd_kernel_dense.hip", "mkd_kernel_moe.hip", "mkd_kernel_batch.hip", "mkd_launch.hip", "mkd_probe.hip"]
HOST_SRCS = ["mkd_api.cpp", "schedule.cpp"]
HEADERS = [os.path.join(CSRC, "mkd_device.h"), os.path.join(CSRC, "mkd_internal.h"),
           os.path.join(INCLUDE, "mkd.h")]


def _steps():
    steps = []
    for src in DEVICE_SRCS:
        steps.append(([HIPCC] + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src)], src, src.rsplit(".", 1)[0] + ".o"))
    steps.append(([HIPCC] + HOST_FLAGS + ["-D__HIP_PLATFORM_AMD__", "-x", "c++", "-c",
                                          os.path.join(CSRC, "mkd_api.cpp")], "mkd_api.cpp", "mkd_api.o"))
    steps.append((["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, "schedule.cpp")], "schedule.cpp", "schedule.o"))
    return steps


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(f) > t for f in [os.path.join(CSRC, src)] + HEADERS)


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every translation unit (in parallel) and link libmkd.so.
    incremental=True recompiles only objects older than their sources."""
    os.makedirs(BUILD, exist_ok=True)
    procs, objs = [], []
    t0 = time.time()
    for cmd, src, obj in _steps():
        out = os.path.join(BUILD, obj)
        objs.append(out)
        if incremental and not _stale(src, out):
            continue
        tmp = out + ".tmp.o"
        procs.append((obj, out, tmp, cmd, subprocess.Popen(cmd + ["-o", tmp], stdout=subprocess.PIPE,
                                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for obj, out, tmp, cmd, pr in procs:
        log, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(log)
            failed.append(obj)
            continue
        os.replace(tmp, out)
        if verbose:
            print(f"[build] {obj} ({time.time() - t0:.1f}s)", flush=True)
    if failed:
        raise RuntimeError("build failed: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB} ({time.time() - t0:.1f}s)", flush=True)
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
