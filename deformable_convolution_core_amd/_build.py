"""Build libdcn_core.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "dcn_core.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "dcn_kernels.hpp"), os.path.join(ROOT, "include", "dcn_core.h")]
LIB = os.path.join(PKG, "libdcn_core.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    """Compile the HIP library (always recompiles)."""
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-o", out + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
