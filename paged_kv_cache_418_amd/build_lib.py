"""Builds libpa.so (the HIP library behind include/pa.h) for gfx950 with hipcc.

Usage: python -m paged_kv_cache_418_amd.build_lib [--verbose]
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["abi.cpp", "block_pool.cpp", "cache_kernels.hip", "decode_kernels.hip", "prefill_kernels.hip",
           "fused_kernels.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 instructions stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs (the softmax rescales them every tile)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    # PA_EXTRA_CFLAGS: extra compiler flags (e.g. -D switches of a variant being measured)
    extra = os.environ.get("PA_EXTRA_CFLAGS", "").split()
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links libpa.so in the package directory."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    # only the pa_* entry points of include/pa.h are exported
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", f"-Wl,--version-script={os.path.join(CSRC, 'libpa.map')}",
           "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
