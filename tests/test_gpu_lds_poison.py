"""Race detection with the LDS-poison debug build (libdbs_poison.so: every
direct-to-LDS load first fills its destination with 0xFF bytes, NaN in the
8- and 16-bit formats and in every scale format).  A fragment or scale read
that ran ahead of its load's wait would see poison instead of the data of an
older stage, so each case runs on both builds through the C ABI and the
outputs must agree bit for bit (and the product build's with the oracle).
The cases walk every ring of the kernels: 256 x 256 and 256 x 64 tiles, more
tiles than CUs, a partial last stage, two- and three-slot rings, chunked and
per-stage MX scales, the packed E2M1 ring beside an 8-bit operand, the FP6
kernel's chunk buffers and stage-blocked operands, the raw NVFP4 stages,
MN-major staging and both release points of the decoupled-ring BF16 kernel."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu
from tests.test_gpu_layouts import run_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def poison():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    return dbs.load_poison_library()


def _same(run, poison, label):
    D = run()
    with dbs.using_library(poison):
        Dp = run()
    torch.cuda.synchronize()
    a, b = _gpu.d_bits(D), _gpu.d_bits(Dp)
    bad = np.argwhere(a != b)
    assert bad.size == 0, f"{label}: {len(bad)} outputs differ under LDS poison, first at {tuple(bad[0])}"
    return D


SHAPES = [
    (300, 520, 352),      # 256 x 64 tiles, partial last stage, register-staged MX scales
    (256, 20000, 512),    # 313 tiles of 256 x 64: a second persistent round, three-slot ring
    (300, 9000, 768),     # raw NVFP4 on 4 waves, three stages a tile
    (3000, 2900, 352),    # 256 x 256, partial last stage
    (5000, 4100, 512),    # 256 x 256 over more than one persistent round, chunked MX scales
    (512, 260, 4096),     # long K
]


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_poison_matches(poison, fmt, shape):
    M, N, K = shape
    _gpu.say(f"[poison] {fmt} {shape}")
    w = synth.workload(fmt, M, N, K, 71, 72)
    d = _gpu.to_dev(w)
    D = _same(lambda: _gpu.run(fmt, w, d), poison, f"{fmt} {shape}")
    if M * N <= 3_000_000:
        _gpu.check_full(fmt, w, D)


@pytest.mark.parametrize("pair,shape", [
    (("e4m3", "e2m1"), (3000, 2900, 512)),     # the E2M1 operand in a ring of its own, 256 x 256
    (("e2m1", "e4m3"), (300, 9000, 768)),      # ... on 256 x 64 tiles
    (("e2m3", "e2m3"), (2900, 3100, 1024)),    # FP6-rate kernel, chunked scales
    (("e3m2", "e4m3"), (300, 520, 352)),       # an FP6 operand widened on its way into LDS
], ids=lambda v: "x".join(map(str, v)))
def test_poison_mixed(poison, pair, shape):
    M, N, K = shape
    _gpu.say(f"[poison] {pair} {shape}")
    w = synth.workload("mxfp8", M, N, K, 73, 74, *pair)
    d = _gpu.to_dev(w)
    _same(lambda: dbs.gemm_mx_mixed(pair[0], pair[1], d["A"], d["sA"], d["B"], d["sB"], K=K), poison,
          f"{pair} {shape}")


@pytest.mark.parametrize("shape", [(2304, 2304, 512), (2301, 2299, 640)], ids=lambda s: "x".join(map(str, s)))
def test_poison_nvfp4_fp6(poison, shape):
    """The FP6-rate kernel on the FP4-rate NVFP4 path's stage-blocked operands
    (chunked scales; per-stage scales and partial row groups)."""
    M, N, K = shape
    _gpu.say(f"[poison] nvfp4_fp6 {shape}")
    w = synth.workload("nvfp4", M, N, K, 79, 80)
    d = _gpu.to_dev(w)
    _same(lambda: dbs.gemm_nvfp4_fp6(d["A"], d["sA"], w["tA"], d["B"], d["sB"], w["tB"]), poison,
          f"nvfp4_fp6 {shape}")


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("lay", [(1, 0), (1, 1)], ids=["mk", "mm"])
def test_poison_mn_major(poison, fmt, lay):
    M, N, K = 2912, 3008, 512      # MN-major rows of whole 16-byte chunks
    _gpu.say(f"[poison] {fmt} layout {lay}")
    w = synth.workload(fmt, M, N, K, 75, 76)
    _same(lambda: run_layout(fmt, w, *lay), poison, f"{fmt} layout {lay}")


@pytest.mark.parametrize("early", [True, False], ids=["early-A", "late-A"])
@pytest.mark.parametrize("shape", [(3000, 2900, 352), (5000, 4100, 128)], ids=lambda s: "x".join(map(str, s)))
def test_poison_decoupled(poison, early, shape):
    M, N, K = shape
    _gpu.say(f"[poison] bf16 decoupled early={early} {shape}")
    w = synth.workload("bf16", M, N, K, 77, 78)
    d = _gpu.to_dev(w)
    _same(lambda: dbs.gemm_bf16_decoupled(d["A"], d["B"], early_release_a=early), poison,
          f"decoupled {early} {shape}")
