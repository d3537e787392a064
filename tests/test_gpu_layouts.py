"""GPU parity of the MN-major operand layouts (A stored K x M, B stored K x N)
through the C ABI.  The operands are the seeded K-major workloads of the other
parity tests, handed to the library transposed (E2M1 re-packed along M or N);
the oracle computes on the K-major codes, so any slip in the staging or the
transposed LDS reads shows up against it."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu
from tests.test_gpu_parity import _identity_w

pytestmark = pytest.mark.gpu

FMTS = ["bf16", "mxfp8", "mxfp4", "nvfp4"]
LAYS = [(1, 0), (0, 1), (1, 1)]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def to_mn(fmt: str, X: np.ndarray) -> np.ndarray:
    """K-major operand storage (rows, K) -> MN-major storage (K, rows)."""
    if fmt in ("bf16", "mxfp8"):
        return np.ascontiguousarray(X.T)
    codes = np.empty((X.shape[0], 2 * X.shape[1]), np.uint8)     # E2M1: unpack along K
    codes[:, 0::2] = X & 0xF
    codes[:, 1::2] = X >> 4
    t = np.ascontiguousarray(codes.T)                             # (K, rows)
    return (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)      # pack along rows


def run_layout(fmt: str, w: dict, la: int, lb: int) -> torch.Tensor:
    A = to_mn(fmt, w["A"]) if la else w["A"]
    B = to_mn(fmt, w["B"]) if lb else w["B"]
    d = _gpu.to_dev({"A": A, "B": B, **({"sA": w["sA"], "sB": w["sB"]} if fmt != "bf16" else {})})
    if fmt == "bf16":
        return dbs.gemm_bf16(d["A"], d["B"], la=la, lb=lb)
    if fmt == "nvfp4":
        return dbs.gemm_nvfp4(d["A"], d["sA"], w["tA"], d["B"], d["sB"], w["tB"], la=la, lb=lb)
    elem = "e4m3" if fmt == "mxfp8" else "e2m1"
    return dbs.gemm_mx(elem, d["A"], d["sA"], d["B"], d["sB"], K=w["K"], la=la, lb=lb)


def _lay_id(l):
    return {(1, 0): "mnA", (0, 1): "mnB", (1, 1): "mnAB"}[l]


# 256 x 64 tiles (the first two) and 256 x 256 tiles (the rest); M and N
# multiples of 32 so that every format's MN-major K-rows are whole 16-byte
# chunks.  K = 352: partial last stage in every format and MX scale rows of
# 11 bytes (register-staged scales); K = 512: whole chunks of stage scales.
SHAPES = [
    (288, 320, 352),
    (256, 19968, 512),     # 312 tiles: several per workgroup
    (2944, 3072, 352),
    (3008, 2944, 512),
    (4128, 4096, 256),     # 17 x 16 = 272 tiles: a second persistent round
]


@pytest.mark.parametrize("lay", LAYS, ids=_lay_id)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layout_matches_oracle(shape, fmt, lay):
    M, N, K = shape
    _gpu.say(f"[layout] {fmt} {_lay_id(lay)} {shape}")
    w = synth.workload(fmt, M, N, K, 700 + M % 97, 800 + N % 89)
    D = run_layout(fmt, w, *lay)
    torch.cuda.synchronize()
    if M * N <= 1 << 23:
        _gpu.check_full(fmt, w, D)
    else:
        em, en = synth.sample_entries(71, M, N, 4096)
        _gpu.check_sampled(fmt, w, D.contiguous(), em, en)


@pytest.mark.parametrize("lay", LAYS, ids=_lay_id)
@pytest.mark.parametrize("fmt", FMTS)
def test_layout_edges(fmt, lay):
    """The smallest MN-major rows each format takes (16 bytes: 8 bf16, 16
    E4M3, 32 E2M1), a single output tile, and K of one MX block."""
    rows = {"bf16": 8, "mxfp8": 16, "mxfp4": 32, "nvfp4": 32}[fmt]
    for M, N, K in [(rows, rows, 32), (rows, 3 * rows, 96), (5 * rows, rows, 64)]:
        _gpu.say(f"[layout] {fmt} {_lay_id(lay)} edge {(M, N, K)}")
        w = synth.workload(fmt, M, N, K, 11, 12)
        D = run_layout(fmt, w, *lay)
        torch.cuda.synchronize()
        _gpu.check_full(fmt, w, D)


@pytest.mark.parametrize("lay", LAYS, ids=_lay_id)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mk", [(288, 512), (3008, 2944)], ids=lambda s: "x".join(map(str, s)))
def test_layout_exact_permutation(fmt, lay, mk):
    """A times a permutation matrix, bit for bit, with either operand MN-major:
    every output is one decoded, scaled element of A."""
    M, K = mk
    _gpu.say(f"[layout] {fmt} {_lay_id(lay)} exact permutation {M}x{K}x{K}")
    w = _identity_w(fmt, M, K, np.random.default_rng(35), True)
    D = run_layout(fmt, w, *lay)
    torch.cuda.synchronize()
    if M * K <= 1 << 20:
        _gpu.check_exact(fmt, w, D)
    else:
        em, en = synth.sample_entries(36, M, K, 4096)
        _gpu.check_exact_sampled(fmt, w, D.contiguous(), em, en)


@pytest.mark.parametrize("fmt", FMTS)
def test_layouts_agree_bitwise(fmt):
    """All four layout combinations give the same bits (the MFMAs see the
    same fragments, whatever the staging).  NVFP4 with an MN-major operand
    runs other kernels than K-major NVFP4 (codes decoded in registers, K
    summed in another grouping), so there the three MN-major combinations
    agree with each other."""
    _gpu.say(f"[layout] {fmt} all layouts agree")
    w = synth.workload(fmt, 2944, 3008, 512, 91, 92)
    lays = LAYS if fmt == "nvfp4" else [(0, 0), *LAYS]
    outs = [_gpu.d_bits(run_layout(fmt, w, la, lb)) for la, lb in lays]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("shape", [(32, 32, 16), (64, 96, 48), (288, 320, 336), (2944, 3072, 1040)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nvfp4_mn_odd_blocks(shape):
    """NVFP4 with both operands MN-major and K an odd multiple of 16: the
    last stage ends halfway through a 32-element half-row, on K-rows and
    scale bytes that read as zero past K."""
    M, N, K = shape
    _gpu.say(f"[layout] nvfp4 mnAB odd K {shape}")
    w = synth.workload("nvfp4", M, N, K, 13 + K % 7, 14 + M % 5)
    D = run_layout("nvfp4", w, 1, 1)
    torch.cuda.synchronize()
    if M * N <= 1 << 23:
        _gpu.check_full("nvfp4", w, D)
    else:
        em, en = synth.sample_entries(73, M, N, 4096)
        _gpu.check_sampled("nvfp4", w, D.contiguous(), em, en)


@pytest.mark.parametrize("lay", LAYS, ids=_lay_id)
def test_nvfp4_mn_scale_rows_unaligned(lay):
    """Scale rows whose base is not dword aligned: the register-staged scale
    path of the MN-major NVFP4 kernels."""
    M, N, K = 288, 320, 512
    _gpu.say(f"[layout] nvfp4 {_lay_id(lay)} unaligned scale rows")
    w = synth.workload("nvfp4", M, N, K, 15, 16)
    A = to_mn("nvfp4", w["A"]) if lay[0] else w["A"]
    B = to_mn("nvfp4", w["B"]) if lay[1] else w["B"]
    d = _gpu.to_dev({"A": A, "B": B})
    sa = torch.zeros(w["sA"].size + 1, dtype=torch.uint8, device="cuda")
    sb = torch.zeros(w["sB"].size + 1, dtype=torch.uint8, device="cuda")
    sa[1:] = torch.from_numpy(w["sA"].reshape(-1)).cuda()
    sb[1:] = torch.from_numpy(w["sB"].reshape(-1)).cuda()
    D = dbs.gemm_nvfp4(d["A"], sa[1:].view(M, K // 16), w["tA"], d["B"], sb[1:].view(N, K // 16), w["tB"],
                       la=lay[0], lb=lay[1])
    torch.cuda.synchronize()
    _gpu.check_full("nvfp4", w, D)
