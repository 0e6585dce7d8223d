"""Build the HIP library libnsa.so in-tree for gfx950 with hipcc.

Usage: python -m top_kv_tile_amd.build   (or top_kv_tile_amd.build.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnsa.so")
SOURCES = ["nsa_api.cpp", "select_kernels.hip", "attn_kernels.hip", "attn_bwd_kernels.hip", "reorder_kernels.hip"]

# Packed fp32 instructions are kept out of the device code: hipcc -O3 would
# otherwise form them from plain float code.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast",
    "-Wno-unused-command-line-argument",
]
# Matrix-core accumulators are kept in ordinary VGPRs (-amdgpu-mfma-vgpr-form)
# rather than AGPRs. The selection kernels needed it; the attention and
# gradient kernels compile to the same code either way (at two waves per
# SIMD their accumulators fit the unified register file).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
PER_SOURCE: dict = {}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnsa.so)")


# hipcc's host pass does not know the packed-fp32 feature and says so; that is expected.
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, what, verbose):
    _, stderr = proc.communicate()
    err = "\n".join(l for l in stderr.splitlines() if _NOISE not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


# Host-side AddressSanitizer build of the C ABI layer (nsa_api.cpp): the
# host pass only (-Xarch_host), the device code unchanged. Load it into a
# process with the compiler's ASan runtime preloaded.
ASAN_LIB = os.path.join(HERE, "libnsa_asan.so")
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, asan: bool = False) -> str:
    """Compile every source (in parallel) and link top_kv_tile_amd/libnsa.so
    (libnsa_asan.so with asan=True); returns the path."""
    include = ["-I", os.path.join(ROOT, "include")]
    lib = ASAN_LIB if asan else LIB
    with tempfile.TemporaryDirectory(prefix="_build_", dir=HERE) as tmpdir:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            flags = PER_SOURCE.get(src, VGPR_FORM)
            extra = ASAN_HOST if (asan and src.endswith(".cpp")) else []
            procs.append((src, _run([hipcc(), *FLAGS, *flags, *extra, *include, "-c", "-o", obj,
                                     os.path.join(CSRC, src)], verbose)))
            objs.append(obj)
        for src, proc in procs:
            _finish(proc, src, verbose)
        tmp = lib + ".tmp"
        link_extra = ["-Xarch_host", "-fsanitize=address"] if asan else []
        _finish(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs], verbose),
                "the link", verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, asan="--asan" in sys.argv[1:]))
