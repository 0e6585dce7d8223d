"""Build the HIP library libnsa.so in-tree for gfx950 with hipcc.

Usage: python -m top_kv_tile_amd.build   (or top_kv_tile_amd.build.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnsa.so")
SOURCES = ["nsa_api.cpp", "select_kernels.hip", "attn_kernels.hip", "attn_bwd_kernels.hip", "reorder_kernels.hip"]

# Packed fp32 instructions are kept out of the device code: hipcc -O3 would
# otherwise form them from plain float code. Matrix-core accumulators are
# allocated as ordinary VGPRs (gfx950 MFMAs take them there): with the default
# AGPR form the register allocator shuttled live dK/dV accumulators between
# AGPRs and VGPRs on every iteration of the gradient kernel.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-ffp-contract=fast",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnsa.so)")


def build(verbose: bool = False) -> str:
    """Compile every source into top_kv_tile_amd/libnsa.so; returns the path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is expected.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
