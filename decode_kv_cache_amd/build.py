"""Build the in-tree HIP libraries for gfx950 with hipcc.

  libkvx.so        the transfer library (C ABI in include/kvx.h)
  libkvx_bench.so  measurement helpers for the bench and GPU tests

Run ``python -m decode_kv_cache_amd.build`` (or ``__graft_entry__.build()``).
Every call compiles from source.
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

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ROCM = os.environ.get("ROCM_PATH") or os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    # packed fp32 instructions off for every device compile
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# plain C++ translation units (no kernels) still include the HIP runtime API
HOST_CXX = [f"-isystem{os.path.join(ROCM, 'include')}", "-D__HIP_PLATFORM_AMD__=1"]

TARGETS = {
    "libkvx.so": ["kvx_host.cpp", "kvx_xfer.cpp", "kvx_queue.cpp", "kvx_kernels.hip"],
    "libkvx_bench.so": ["kvx_bench_support.hip"],
}


def lib_path(name: str) -> str:
    return os.path.join(PKG, name)


def _compile(out: str, sources, verbose: bool) -> None:
    tmp = out + f".tmp{os.getpid()}"
    srcs = []
    for s in sources:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".hip") else HOST_CXX + ["-x", "c++", p])
    cmd = [HIPCC] + COMMON + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if r.stderr.strip() and verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> None:
    for name, sources in TARGETS.items():
        _compile(lib_path(name), sources, verbose)


if __name__ == "__main__":
    build(verbose=True)
