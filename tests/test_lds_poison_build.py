"""Structure of the LDS-poison debug build (no GPU): every kernel unit that
stages through direct-to-LDS loads is compiled for gfx950 with
DBS_LDS_POISON=1, and in its assembly every such load (`buffer_load_dword*
... lds`) must come after a poison write (`ds_write`) that an
`s_waitcnt lgkmcnt(0)` has waited for, with no other direct-to-LDS load in
between, and the product build must hold the same number of direct-to-LDS
loads.  The GPU side
(tests/test_gpu_lds_poison.py) then compares the two builds' results bit for
bit."""
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "dense_block_scaled_amd" / "csrc"
HIPCC = "/opt/rocm/bin/hipcc"
UNITS = ["gemm_bf16.hip", "gemm_mxfp4.hip", "gemm_mxfp6.hip", "gemm_bf16_ea.hip", "gemm_nvfp4.hip"]
DMA = re.compile(r"^\s*buffer_load_dword\S*\s.*\blds\b")


def _asm(unit: str, poison: bool, out: Path) -> str:
    dst = out / (unit + (".poison.s" if poison else ".s"))
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", f"-I{ROOT / 'include'}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           *(["-DDBS_LDS_POISON=1"] if poison else []), str(CSRC / unit), "-o", str(dst)]
    subprocess.run(cmd, check=True, capture_output=True)
    return dst.read_text()


def _check(text: str) -> tuple[int, int]:
    """(direct-to-LDS loads, those preceded by a waited-for poison write)"""
    n = guarded = 0
    wrote = waited = False
    for line in text.splitlines():
        s = line.strip()
        if not s or s.startswith(";") or s.startswith("."):
            continue
        if DMA.match(line):
            n += 1
            guarded += wrote and waited
            wrote = waited = False
        elif s.startswith("ds_write"):
            wrote, waited = True, False
        elif s.startswith("s_waitcnt") and "lgkmcnt(0)" in s and wrote:
            waited = True
    return n, guarded


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    if not Path(HIPCC).exists():
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("poison_asm")
    jobs = [(u, p) for u in UNITS for p in (False, True)]
    with ThreadPoolExecutor(max_workers=8) as pool:
        texts = list(pool.map(lambda j: _asm(j[0], j[1], out), jobs))
    return {j: t for j, t in zip(jobs, texts)}


@pytest.mark.parametrize("unit", UNITS)
def test_every_lds_load_is_poisoned_first(listings, unit):
    n, guarded = _check(listings[(unit, True)])
    assert n > 0, f"{unit}: no direct-to-LDS loads found"
    assert guarded == n, f"{unit}: {n - guarded} of {n} direct-to-LDS loads lack a waited-for poison write"
    n_prod, _ = _check(listings[(unit, False)])
    assert n_prod == n, f"{unit}: {n_prod} direct-to-LDS loads in the product build, {n} in the poison build"
