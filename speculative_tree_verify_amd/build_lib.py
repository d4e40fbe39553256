"""Build libstv.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libstv.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("stv_kernels.hip", "stv_accept.hip", "stv_lookup.hip", "stv_abi.cpp")]
ARCH = "gfx950"

# Packed fp32 VALU forms stay off: float code is compiled to scalar-lane ops.
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA accumulators live in VGPRs, so the VALU softmax rescale needs no
             # AGPR round trips
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), *HIP_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    print(LIB_PATH)
    sys.exit(0)
