"""Every read of an MFMA result in the gfx950 kernels comes after the wait
states the CDNA ISA requires (number of passes + 3: 19 for the 16-pass MFMAs
-- 32x32x16 f8 forms and the scaled f8f6f4 MFMA with an 8-bit operand -- and
11 for the 8-pass ones), on every control path of the compiled code.

The check compiles each kernel translation unit to gfx950 assembly with the
library's own flags (no GPU needed) and walks, from every MFMA, all paths
(fall-through and branch targets) to the first non-MFMA instruction reading
one of its destination registers, counting one wait state per instruction
and N + 1 per `s_nop N`.  An accumulating MFMA that takes the same registers
as its C operand is a new producer, not a reader.  Empty inline-asm
statements issue nothing, so they count as zero here; the compiler's hazard
recognizer counts them as one each, which is why the kernels keep them away
from MFMA results."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "dense_block_scaled_amd" / "csrc"
UNITS = ["gemm_bf16.hip", "gemm_mxfp8.hip", "gemm_mx8_e5m2.hip", "gemm_mx8_fp4.hip", "gemm_mxfp4.hip",
         "gemm_nvfp4.hip", "gemm_mxfp6.hip", "gemm_bf16_ea.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def required_wait_states(op, ops):
    """passes + 3 for an MFMA mnemonic (None for anything else)."""
    if op.startswith("v_mfma_scale_f32_32x32x64_f8f6f4"):
        codes = dict(o.split(":") for o in ops if o.startswith(("cbsz:", "blgp:")))
        a, b = int(codes.get("cbsz", 0)), int(codes.get("blgp", 0))
        return 19 if (a <= 1 or b <= 1) else 11      # an 8-bit operand: 16 passes
    if op.startswith("v_mfma_scale_f32_16x16x128_f8f6f4"):
        codes = dict(o.split(":") for o in ops if o.startswith(("cbsz:", "blgp:")))
        a, b = int(codes.get("cbsz", 0)), int(codes.get("blgp", 0))
        return 11 if (a <= 1 or b <= 1) else 7
    if op.startswith("v_mfma_f32_32x32x16_") or op.startswith("v_mfma_f32_32x32x8"):
        return 11
    if op.startswith("v_mfma_f32_16x16x32_"):
        return 7
    if op.startswith("v_mfma"):
        return 19                                    # anything else: the longest
    return None


def scan(asm_text):
    """(paths checked, list of (gap, need, mfma, reader)) for one assembly file."""
    lines = []
    for raw in asm_text.splitlines():
        s = raw.split(";")[0].strip()
        if not s or (s.startswith(".") and not s.endswith(":")):
            continue
        lines.append(s)
    label = {s[:-1]: i for i, s in enumerate(lines) if s.endswith(":")}
    short, checked = [], 0
    for i, s in enumerate(lines):
        if s.endswith(":"):
            continue
        parts = s.replace(",", " ").split()
        need = required_wait_states(parts[0], parts[1:])
        if need is None:
            continue
        dst = _regs(parts[1])
        stack, seen, worst = [(i + 1, 0)], {}, None
        while stack:
            j, ws = stack.pop()
            while j < len(lines) and ws < need + 8:
                t = lines[j]
                if t.endswith(":"):
                    j += 1
                    continue
                if seen.get(j, 1 << 30) <= ws:
                    break
                seen[j] = ws
                p = t.replace(",", " ").split()
                op, a = p[0], p[1:]
                if op == "s_nop":
                    ws += int(a[0]) + 1
                    j += 1
                    continue
                if op.startswith("v_mfma"):
                    if dst & (_regs(a[1]) | _regs(a[2])):
                        if worst is None or ws < worst:
                            worst, short_reader = ws, t
                        break
                    if _regs(a[0]) & dst:
                        break                        # accumulates in place: a new producer
                    ws += 1
                    j += 1
                    continue
                reads = set()
                stores = op.startswith(("buffer_store", "global_store", "ds_write", "scratch_store", "v_accvgpr_read"))
                for tk in (a if stores else a[1:]):
                    reads |= _regs(tk)
                if dst & reads:
                    if worst is None or ws < worst:
                        worst, short_reader = ws, t
                    break
                if a and (dst & _regs(a[0])):
                    break                            # overwritten before any read
                if op == "s_branch":
                    j = label[a[0]]
                    continue
                if op.startswith("s_cbranch"):
                    stack.append((label[a[0]], ws + 1))
                if op in ("s_endpgm", "s_setpc_b64"):
                    break
                ws += 1
                j += 1
        if worst is not None:
            checked += 1
            if worst < need:
                short.append((worst, need, s, short_reader))
    return checked, short


def _compile(unit, outdir):
    out = Path(outdir) / (unit + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", f"-I{ROOT / 'include'}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           str(CSRC / unit), "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out.read_text()


def test_scanner_flags_a_short_gap():
    """The scan itself: a read two instructions after a 16-pass MFMA is short,
    the same read behind s_nop 15 / s_nop 3 is not, and an empty inline-asm
    marker counts for nothing."""
    mf = "v_mfma_scale_f32_32x32x64_f8f6f4 v[2:17], v[2:9], v[10:17], 0, v1, v18 op_sel_hi:[0,0,0]"
    bad = f"k:\n\t{mf}\n\t;;#ASMSTART\n\t;;#ASMEND\n\tv_mov_b32 v40, 0\n\tv_fmamk_f32 v1, v2, 0x40400000, v7\n"
    good = f"k:\n\t{mf}\n\ts_nop 15\n\ts_nop 3\n\tv_fmamk_f32 v1, v2, 0x40400000, v7\n"
    assert scan(bad)[1] and scan(bad)[1][0][:2] == (1, 19)
    assert scan(good) == (1, [])
    f4 = mf + " cbsz:4 blgp:4"
    assert scan(f"k:\n\t{f4}\n\ts_nop 10\n\tv_fmamk_f32 v1, v2, 0x40400000, v7\n") == (1, [])


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")
def test_every_mfma_result_read_waits_long_enough():
    tmp = tempfile.mkdtemp(prefix="dbs_asm_")
    try:
        with ThreadPoolExecutor(max_workers=min(len(UNITS), os.cpu_count() or 1)) as pool:
            texts = list(pool.map(lambda u: _compile(u, tmp), UNITS))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    total = 0
    for unit, text in zip(UNITS, texts):
        checked, short = scan(text)
        total += checked
        assert not short, f"{unit}: {len(short)} MFMA results read too early, e.g. {short[0]}"
    assert total > 1000       # the scan saw the epilogue reads of every kernel
