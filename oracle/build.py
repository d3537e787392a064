"""Builds oracle/liboracle.so from oracle.c with the host C compiler.

Test infrastructure: compiled by ``__graft_entry__.build()`` and on first use
by the tests.  No GPU code, no shared source with the HIP library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from pathlib import Path

HERE = Path(__file__).resolve().parent


def build(verbose: bool = False) -> Path:
    src = HERE / "oracle.c"
    out = HERE / "liboracle.so"
    # build into a temp name then rename, so a concurrent loader never sees a
    # half-written library
    fd, tmp = tempfile.mkstemp(prefix="liboracle.", suffix=".so.tmp", dir=str(HERE))
    os.close(fd)
    cmd = [os.environ.get("CC", "gcc"), "-std=c11", "-O2", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-pthread",
           str(src), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
