"""Build libbsattn.so (and the benchmark's libbsattn_probe.so) in-tree with
hipcc for gfx950.

    python -m block_sparse_flash_bsa_amd.build          # build (always recompiles)

Every HIP source is compiled with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
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
LIB = os.path.join(PKG, "libbsattn.so")
PROBE_LIB = os.path.join(PKG, "libbsattn_probe.so")   # benchmark's MFMA-rate probe
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

SOURCES = ["plan.cpp", "plan_device.hip", "forward.hip", "backward.hip", "merge.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsattn)")


def build(verbose: bool = False) -> str:
    """Compile every source and link libbsattn.so next to this file."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        if src.endswith(".hip"):
            cmd = [cc, *COMMON, *HIP_FLAGS, "-x", "hip"]
        else:  # host-only C++ (HIP runtime API, no device code)
            cmd = [cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE]
        cmd += ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    # The benchmark's MFMA throughput probe, a library of its own.
    pobj = os.path.join(objdir, "probe.hip.o")
    cmd = [cc, *COMMON, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, "probe.hip"), "-o", pobj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    ptmp = PROBE_LIB + ".tmp"
    subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", pobj, "-o", ptmp], check=True)
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv[1:]))
