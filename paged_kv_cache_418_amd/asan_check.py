"""AddressSanitizer build of the host code, and the CPU test suite run under it.

The library's host sources (abi.cpp: argument checks, planning, workspace layout;
block_pool.cpp: the host block pool) and the CPU oracle (oracle/pa_oracle.c) are
compiled with AddressSanitizer by gcc; the HIP kernel sources are compiled as in
the normal build (device code is not instrumented).  The results are separate
files in the build folder (libpa_asan.so, liboracle_asan.so), picked up through
PA_LIBRARY / ORACLE_LIBRARY, so the normal build is left alone.  The test run
preloads gcc's ASan runtime and uses no GPU.

Usage: python -m paged_kv_cache_418_amd.asan_check [--build-only] [pytest args ...]
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build_lib

PKG = build_lib.PKG
ROOT = build_lib.ROOT
LIB = os.path.join(build_lib.BUILD, "libpa_asan.so")
ORACLE_SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")
ORACLE_LIB = os.path.join(build_lib.BUILD, "liboracle_asan.so")
HOST_SOURCES = ["abi.cpp", "block_pool.cpp"]
KERNEL_SOURCES = [s for s in build_lib.SOURCES if s.endswith(".hip")]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address", "-fno-omit-frame-pointer", "-g"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed:\n{r.stdout}{r.stderr}")


def build() -> tuple:
    """Builds libpa_asan.so and liboracle_asan.so; returns their paths."""
    os.makedirs(build_lib.BUILD, exist_ok=True)
    objs = [build_lib._compile(s, False) for s in KERNEL_SOURCES]
    for src in HOST_SOURCES:
        obj = os.path.join(build_lib.BUILD, "asan_" + os.path.splitext(src)[0] + ".o")
        _run(["g++", "-std=c++17", "-O1", "-fPIC", "-Wall", *SAN, "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include", f"-I{build_lib.INCLUDE}", f"-I{build_lib.CSRC}", "-c",
              os.path.join(build_lib.CSRC, src), "-o", obj])
        objs.append(obj)
    _run(["g++", "-shared", *SAN, "-o", LIB, *objs, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    _run(["gcc", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          "-Wall", *SAN, "-o", ORACLE_LIB, ORACLE_SRC, "-lm"])
    return LIB, ORACLE_LIB


def asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def main(argv) -> int:
    build()
    if "--build-only" in argv:
        print(LIB, ORACLE_LIB)
        return 0
    extra = [a for a in argv if a != "--build-only"]
    env = dict(os.environ, PA_LIBRARY=LIB, ORACLE_LIBRARY=ORACLE_LIB, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-x", *extra]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
