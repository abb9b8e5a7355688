"""Build libgqa_decode.so in-tree for gfx950 with hipcc.

    python -m gqa_split_kv_amd.build        (or build() from Python)

Every HIP source is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the host-only C++ (plan.cpp) is compiled
without it.  Objects go to gqa_split_kv_amd/_build/, the library to
gqa_split_kv_amd/libgqa_decode.so.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa_decode.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
DEVICE_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The sweep kernel's instruction schedule: LLVM's max-ilp strategy measured
# 0.25-0.7% faster than the default on every decode form (bit-identical code paths).
SWEEP_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    # Device + host code of the kernels.
    for name in ("sweep_kernel", "merge_kernel"):
        src = os.path.join(CSRC, name + ".hip")
        obj = os.path.join(BUILD, name + ".o")
        extra = SWEEP_FLAGS if name == "sweep_kernel" else []
        _run([HIPCC, "-x", "hip", "--offload-arch=" + ARCH, *COMMON, *NO_PACKED_FP32, *DEVICE_FLAGS, *extra,
              "-c", src, "-o", obj], verbose)
        objs.append(obj)
    # Prefill kernel: its accumulators live in AGPRs (no VGPR-form MFMA).
    src = os.path.join(CSRC, "prefill_kernel.hip")
    obj = os.path.join(BUILD, "prefill_kernel.o")
    _run([HIPCC, "-x", "hip", "--offload-arch=" + ARCH, *COMMON, *NO_PACKED_FP32, "-c", src, "-o", obj],
         verbose)
    objs.append(obj)
    # Measurement probes (plain copy / read kernels).
    src = os.path.join(CSRC, "probe_kernels.hip")
    obj = os.path.join(BUILD, "probe_kernels.o")
    _run([HIPCC, "-x", "hip", "--offload-arch=" + ARCH, *COMMON, *NO_PACKED_FP32, "-c", src, "-o", obj],
         verbose)
    objs.append(obj)
    # C ABI layer: HIP runtime host API only.
    src = os.path.join(CSRC, "api.cpp")
    obj = os.path.join(BUILD, "api.o")
    _run([HIPCC, "-x", "hip", "--offload-arch=" + ARCH, *COMMON, *NO_PACKED_FP32, "-c", src, "-o", obj],
         verbose)
    objs.append(obj)
    # Pure host C++ (validation and planning).
    src = os.path.join(CSRC, "plan.cpp")
    obj = os.path.join(BUILD, "plan.o")
    _run(["g++", *COMMON, "-c", src, "-o", obj], verbose)
    objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
