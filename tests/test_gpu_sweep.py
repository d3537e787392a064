"""Seeded sweep of GPU parity cases over formats, operand layouts and element
mixes at ragged shapes (every output against the oracle).  Shapes are drawn
per case from PCG64(case seed): M, N up to 700 (multiples of what MN-major
rows need when a layout is MN-major), K up to 1024 in the format's
granularity."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu
from tests.test_gpu_layouts import to_mn

pytestmark = pytest.mark.gpu

# (format, element pair for 8-bit MX ("mn": NVFP4 with an MN-major operand),
#  K granularity, MN-major row granularity or None)
KINDS = [
    ("bf16", None, 8, 8),
    ("mxfp8", ("e4m3", "e4m3"), 32, 16),
    ("mxfp8", ("e5m2", "e4m3"), 32, None),
    ("mxfp8", ("e4m3", "e5m2"), 32, None),
    ("mxfp8", ("e5m2", "e5m2"), 32, None),
    ("mxfp4", None, 32, 32),
    ("nvfp4", None, 16, None),
    ("nvfp4", "mn", 16, 32),
    ("mxfp8", ("e5m2", "e4m3"), 32, 16),          # E5M2 pairs take MN-major operands
    ("mxfp8", ("e4m3", "e2m1"), 256, 32),         # FP8 x FP4 packed path (K % 256 == 0), any layout
    ("mxfp8", ("e2m1", "e5m2"), 256, 32),
    ("mxfp8", ("e2m3", "e3m2"), 32, None),       # FP6 (widened, K-major)
    ("mxfp8", ("e3m2", "e4m3"), 32, None),
]
CASES = [(i, k) for k in range(len(KINDS)) for i in range(6)]


def _draw(seed, kgran, mngran, mn_only=False):
    g = np.random.Generator(np.random.PCG64(seed))
    lay = (int(g.integers(0, 2)), int(g.integers(0, 2))) if mngran else (0, 0)
    if mn_only and lay == (0, 0):
        lay = (1, 1)
    def dim(mn):
        if mn and mngran:
            return int(g.integers(1, 700 // mngran + 1)) * mngran
        return int(g.integers(1, 701))
    M, N = dim(lay[0]), dim(lay[1])
    K = int(g.integers(1, 1024 // kgran + 1)) * kgran
    if mn_only and lay != (1, 1) and K % 32:
        K += 16        # NVFP4 with one K-major operand: whole 32-element half-rows
    return M, N, K, lay


@pytest.mark.parametrize("case,kind", CASES, ids=lambda v: str(v))
def test_sweep(case, kind):
    fmt, pair, kgran, mngran = KINDS[kind]
    M, N, K, lay = _draw(1000 * kind + case, kgran, mngran, pair == "mn")
    _gpu.say(f"[sweep] {fmt} {pair or ''} M={M} N={N} K={K} layouts={lay}")
    if pair == "mn":
        pair = None
    if pair:
        w = synth.workload(fmt, M, N, K, 3 * case + 1, 3 * case + 2, *pair)
    else:
        w = synth.workload(fmt, M, N, K, 3 * case + 1, 3 * case + 2)
    ea, eb = pair if pair else (None, None)
    A = to_mn("mxfp4" if ea == "e2m1" else fmt, w["A"]) if lay[0] else w["A"]
    B = to_mn("mxfp4" if eb == "e2m1" else fmt, w["B"]) if lay[1] else w["B"]
    d = _gpu.to_dev({"A": A, "B": B, **({"sA": w["sA"], "sB": w["sB"]} if fmt != "bf16" else {})})
    if fmt == "bf16":
        D = dbs.gemm_bf16(d["A"], d["B"], la=lay[0], lb=lay[1])
    elif fmt == "nvfp4":
        D = dbs.gemm_nvfp4(d["A"], d["sA"], w["tA"], d["B"], d["sB"], w["tB"], la=lay[0], lb=lay[1])
    else:
        ea, eb = pair if pair else ("e2m1", "e2m1")
        D = dbs.gemm_mx_mixed(ea, eb, d["A"], d["sA"], d["B"], d["sB"], K=K, la=lay[0], lb=lay[1])
    torch.cuda.synchronize()
    _gpu.check_full(fmt, w, D)
