"""Build libkvcopy.so (HIP, gfx950) in-tree.

Host C++ (planner, runtime) is compiled with g++ against the HIP runtime
headers; the kernel file with hipcc for gfx950; hipcc links the shared
library.  ``python -m block_copy_amd.build`` runs it from the command line.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libkvcopy.so")
# Measurement-only library: the synthetic decode loop (bf16 GEMV chain) that
# co-runs with copy bursts in the interference benchmark, and the scattered
# read-only and write-only passes that bound the D2D copy.
LOAD_OUT = os.path.join(PKG, "libkvload.so")
LOAD_SOURCES = ["gemv_load.hip", "hbm_probe.hip"]
# Measurement-only program: kvcopy_batch's per-call latency from a C caller.
LATENCY_OUT = os.path.join(PKG, "kvcopy_latency")
BUILD_DIR = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HOST_SOURCES = ["plan.cpp", "runtime.cpp", "jobs.cpp", "autotune.cpp"]
HIP_SOURCES = ["kvcopy_kernel.hip", "device_batch.hip", "order_kernel.hip"]
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Keep the compiler away from packed fp32 instructions on this target.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {cmd[0]} ({r.returncode})")
    return r


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}", "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
              os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    load_objs = []
    for src in LOAD_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        load_objs.append(obj)
    tmp = LOAD_OUT + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *load_objs, "-o", tmp])
    os.replace(tmp, LOAD_OUT)
    tmp = LATENCY_OUT + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
          f"-I{ROCM}/include", f"-I{INCLUDE}", os.path.join(CSRC, "latency_tool.cpp"), "-o", tmp,
          f"-L{PKG}", "-lkvcopy", f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN",
          f"-Wl,-rpath,{os.path.realpath(os.path.join(ROCM, 'lib'))}"])
    os.replace(tmp, LATENCY_OUT)
    if verbose:
        print(f"built {OUT}, {LOAD_OUT} and {LATENCY_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
