"""Builds dense_block_scaled_amd/libdbs.so (the C-ABI library) for gfx950.

    python -m dense_block_scaled_amd.build

hipcc compiles the kernel translation units (csrc/gemm_*.hip: one per group
of formats, all instantiating the template in csrc/gemm_kernel.h), the
launcher (csrc/gemm.hip), the quantisers (csrc/quant.hip) and the ABI layer
(csrc/dbs.cpp) to objects in parallel, then links them, in-tree; no GPU is
needed to build.  Packed-fp32 VALU instructions are turned off for the
device code.  build(poison=True) builds the same sources with
DBS_LDS_POISON=1 into libdbs_poison.so, a debug library whose direct-to-LDS
loads first fill their destination with 0xFF (see gemm_kernel.h); the
race-detection tests compare its results with libdbs.so's bit for bit.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libdbs.so"
POISON_LIB = PKG / "libdbs_poison.so"
ARCH = os.environ.get("DBS_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# largest first, so the longest compile starts first
SOURCES = ["gemm_mx8_fp4.hip", "gemm_mxfp8.hip", "gemm_mx8_e5m2.hip", "gemm_nvfp4.hip", "gemm_mxfp4.hip", "gemm_mxfp6.hip",
           "gemm_bf16.hip", "gemm_bf16_ea.hip", "quant.hip", "gemm.hip", "scratch.hip", "dbs.cpp"]


def _jobs() -> int:
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return max(1, min(n, len(SOURCES), int(os.environ.get("MAX_JOBS", n))))


def build(verbose: bool = False, extra: list[str] | None = None, poison: bool = False) -> Path:
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             f"-I{ROOT / 'include'}", f"-I{CSRC}", *DEVICE_FLAGS, *(["-DDBS_LDS_POISON=1"] if poison else []),
             *(extra or [])]
    out = POISON_LIB if poison else LIB
    objdir = Path(tempfile.mkdtemp(prefix="libdbs.obj.", dir=str(PKG)))
    fd, tmp = tempfile.mkstemp(prefix="libdbs.", suffix=".so.tmp", dir=str(PKG))
    os.close(fd)

    def compile_one(name: str) -> Path:
        obj = objdir / (name + ".o")
        cmd = [HIPCC, *flags, "-c", str(CSRC / name), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    try:
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[str(o) for o in objs], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
        shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, poison=True)
