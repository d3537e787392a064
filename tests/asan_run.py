"""AddressSanitizer run of the CPU test suite (host code only).

    python tests/asan_run.py

Copies the repository to a temporary folder, builds there the C-ABI library
and its LDS-poison debug build with their host code instrumented (each translation unit through hipcc with the
sanitizer flags on the host side only; the gfx950 device code is built as
usual) and the C oracle with the sanitizer, and runs `pytest -m "not gpu"`
against those builds with the sanitizer runtime preloaded.  Exits with
pytest's status; a sanitizer report aborts the process that hit it.  Needs no
GPU; not part of the test suite itself (it runs the suite).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def main() -> int:
    tmp = Path(tempfile.mkdtemp(prefix="dbs_asan_"))
    try:
        repo = tmp / "repo"
        shutil.copytree(ROOT, repo, ignore=shutil.ignore_patterns(".git", "_work", "gpurun_out", "*.so",
                                                                   "__pycache__", "libdbs.obj.*"))
        sys.path.insert(0, str(repo))
        from dense_block_scaled_amd import build as b
        csrc = repo / "dense_block_scaled_amd" / "csrc"
        flags = [f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", f"-I{repo / 'include'}",
                 f"-I{csrc}", *b.DEVICE_FLAGS, *HOST_ASAN]

        def one(job):
            name, poison = job
            obj = tmp / (name + (".poison.o" if poison else ".o"))
            subprocess.run([HIPCC, *flags, *(["-DDBS_LDS_POISON=1"] if poison else []), "-c", str(csrc / name),
                            "-o", str(obj)], check=True)
            return obj

        # the product library and the LDS-poison debug build, both with instrumented host code
        for poison, lib in ((False, "libdbs.so"), (True, "libdbs_poison.so")):
            with ThreadPoolExecutor(max_workers=min(len(b.SOURCES), os.cpu_count() or 1)) as pool:
                objs = list(pool.map(one, [(n, poison) for n in b.SOURCES]))
            subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *HOST_ASAN, *map(str, objs), "-o",
                            str(repo / "dense_block_scaled_amd" / lib)], check=True)
        subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address",
                        "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-pthread",
                        str(repo / "oracle" / "oracle.c"), "-o", str(repo / "oracle" / "liboracle.so"), "-lm"],
                       check=True)
        asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True,
                              text=True).stdout.strip()
        env = dict(os.environ, LD_PRELOAD=asan,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:protect_shadow_gap=0:verify_asan_link_order=0")
        cmd = [sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
               "--deselect", "tests/test_asm_hazards.py::test_every_mfma_result_read_waits_long_enough"]
        return subprocess.run(cmd, cwd=repo, env=env).returncode
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    sys.exit(main())
