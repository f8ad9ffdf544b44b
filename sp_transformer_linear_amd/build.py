"""Build libsptl.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m sp_transformer_linear_amd.build

Compiles every source under csrc/ with hipcc for --offload-arch=gfx950 into _build/ and links
sp_transformer_linear_amd/libsptl.so.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsptl.so")
ARCH = "gfx950"

SOURCES = ["sptl_abi.cpp", "sptl_stager.cpp", "sptl_gemm.hip", "sptl_epilogue.hip", "sptl_noalloc.hip", "sptl_copy.hip", "sptl_affinity.cpp"]

# packed-fp32 instructions are disabled for all device code (the compiler would otherwise
# form them from ordinary float code).
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append(([hipcc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(min(len(jobs), 8)) as ex:
        list(ex.map(lambda j: _run(j[0]), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs], "-o", tmp,
          "-lhsa-runtime64", "-lpthread"])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
