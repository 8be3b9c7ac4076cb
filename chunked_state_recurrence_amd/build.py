"""Build libgla.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m chunked_state_recurrence_amd.build

Compiles ``csrc/gla_kernels.hip``, ``csrc/gla_bwd.hip``, ``csrc/gla_gdn.hip`` and
``csrc/gla_api.hip`` with hipcc into
``chunked_state_recurrence_amd/libgla.so``.  Packed fp32 VALU instructions
are disabled for the device code.
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
LIB = os.path.join(PKG, "libgla.so")
SOURCES = [os.path.join(CSRC, f) for f in ("gla_kernels.hip", "gla_bwd.hip", "gla_gdn.hip", "gla_api.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libgla.so")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-shared", "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
