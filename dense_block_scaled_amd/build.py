"""Builds dense_block_scaled_amd/libdbs.so (the C-ABI library) for gfx950.

    python -m dense_block_scaled_amd.build

hipcc compiles the kernels (csrc/gemm.hip, csrc/quant.hip) and the ABI layer (csrc/dbs.cpp)
in-tree; no GPU is needed to build.  Packed-fp32 VALU instructions are turned
off for the device code.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libdbs.so"
ARCH = os.environ.get("DBS_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    fd, tmp = tempfile.mkstemp(prefix="libdbs.", suffix=".so.tmp", dir=str(PKG))
    os.close(fd)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", f"-I{ROOT / 'include'}", f"-I{CSRC}",
           *DEVICE_FLAGS, *(extra or []),
           str(CSRC / "gemm.hip"), str(CSRC / "quant.hip"), str(CSRC / "dbs.cpp"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
