"""GPU parity of the MX element formats per operand (E4M3 / E5M2 in any
pairing, and either with E2M1: gemm_mx_mixed, gemm_mx('e5m2')) through the C
ABI, against the oracle's per-operand decoding."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu, _pins
from tests.test_gpu_layouts import to_mn

pytestmark = pytest.mark.gpu

PAIRS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3"),
         ("e4m3", "e2m1"), ("e2m1", "e4m3"), ("e5m2", "e2m1"), ("e2m1", "e5m2")]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def run_mixed(w: dict) -> torch.Tensor:
    d = _gpu.to_dev(w)
    ea, eb = w["elemA"], w["elemB"]
    if ea == eb:
        return dbs.gemm_mx(ea, d["A"], d["sA"], d["B"], d["sB"], K=w["K"])
    return dbs.gemm_mx_mixed(ea, eb, d["A"], d["sA"], d["B"], d["sB"], K=w["K"])


def _pid(p):
    return f"{p[0]}x{p[1]}"


# 256 x 64 tiles: register-staged scales (K = 352) and the three-slot ring
# (K = 512); 256 x 256 tiles: register-staged (352), per-stage (384) and
# chunked (512) scales.
SHAPES = [(300, 520, 352), (256, 20000, 512), (3000, 2900, 352), (2900, 3000, 384), (2944, 3008, 512)]


@pytest.mark.parametrize("pair", PAIRS, ids=_pid)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mixed_matches_oracle(shape, pair):
    M, N, K = shape
    _gpu.say(f"[mixed] {_pid(pair)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 500 + M % 53, 600 + N % 59, *pair)
    D = run_mixed(w)
    torch.cuda.synchronize()
    if M * N <= 1 << 23:
        _gpu.check_full("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(72, M, N, 4096)
        _gpu.check_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("pair", PAIRS, ids=_pid)
def test_mixed_random_codes(pair):
    """Codes over each format's whole finite range with random non-unit scales."""
    _gpu.say(f"[mixed] {_pid(pair)} random codes")
    w = _pins.make_w_mx8(*pair, 300, 280, 128, np.random.default_rng(23), scale_lo=112, scale_hi=142)
    D = run_mixed(w)
    torch.cuda.synchronize()
    _gpu.check_full("mxfp8", w, D)


@pytest.mark.parametrize("pair", PAIRS, ids=_pid)
@pytest.mark.parametrize("mk", [(300, 512), (3000, 2944)], ids=lambda s: "x".join(map(str, s)))
def test_mixed_exact_permutation(pair, mk):
    """A (elem_a codes, random scales) times a permutation matrix in elem_b
    with non-unit scales: every output is one decoded element of A times two
    powers of two, exact in bf16, compared bit for bit."""
    M, K = mk
    ea, eb = pair
    _gpu.say(f"[mixed] {_pid(pair)} exact permutation {M}x{K}x{K}")
    rng = np.random.default_rng(39)
    N = K
    w = _pins.make_w_mx8(ea, eb, M, N, K, rng, scale_lo=110, scale_hi=140)
    pi = rng.permutation(K)
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), pi] = {"e5m2": 0x3C, "e4m3": 0x38, "e2m1": 0x2}[eb]   # 1.0
    if eb == "e2m1":
        B = (B[:, 0::2] | (B[:, 1::2] << 4)).astype(np.uint8)
    w["B"] = B
    w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    D = run_mixed(w)
    torch.cuda.synchronize()
    if M * K <= 1 << 20:
        _gpu.check_exact("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(40, M, N, 4096)
        _gpu.check_exact_sampled("mxfp8", w, D, em, en)


def test_grouped_e5m2():
    """The grouped MX GEMM with E5M2 elements on both sides."""
    sizes, N, K = [0, 130, 257, 40], 200, 512
    _gpu.say(f"[mixed] grouped e5m2 sizes={sizes}")
    G, M = len(sizes), int(sum(sizes))
    w = synth.workload("mxfp8", M, G * N, K, 61, 62, "e5m2", "e5m2")
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    d = _gpu.to_dev(w)
    D = dbs.gemm_grouped_mx("e5m2", d["A"], d["sA"], d["B"].reshape(G, N, -1), d["sB"].reshape(G, N, -1),
                            off.tolist(), K=K)
    torch.cuda.synchronize()
    for g in range(G):
        a, b = int(off[g]), int(off[g + 1])
        if a == b:
            continue
        wg = {"fmt": "mxfp8", "M": b - a, "N": N, "K": K, "elemA": "e5m2", "elemB": "e5m2",
              "A": w["A"][a:b], "sA": w["sA"][a:b], "B": w["B"][g * N:(g + 1) * N], "sB": w["sB"][g * N:(g + 1) * N]}
        _gpu.check_full("mxfp8", wg, D[a:b])


def test_e4m3_pair_unchanged():
    """gemm_mx_mixed('e4m3', 'e4m3') is the MXFP8 GEMM, bit for bit."""
    _gpu.say("[mixed] e4m3 x e4m3 via gemm_mx_mixed")
    w = synth.workload("mxfp8", 2944, 3008, 512, 63, 64)
    d = _gpu.to_dev(w)
    D0 = dbs.gemm_mx("e4m3", d["A"], d["sA"], d["B"], d["sB"], K=512)
    D1 = dbs.gemm_mx_mixed("e4m3", "e4m3", d["A"], d["sA"], d["B"], d["sB"], K=512)
    torch.cuda.synchronize()
    assert np.array_equal(_gpu.d_bits(D0), _gpu.d_bits(D1))


E5M2_PAIRS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]
LAYS = [(1, 0), (0, 1), (1, 1)]
# 256 x 64 tiles with register-staged (K = 352) and stage scales (K = 512,
# three-slot ring); 256 x 256 tiles with register-staged (352) and chunked (512)
LAYOUT_SHAPES = [(288, 320, 352), (256, 19968, 512), (2944, 3072, 352), (3008, 2944, 512)]


def _lid(l):
    return {(0, 0): "kk", (1, 0): "mnA", (0, 1): "mnB", (1, 1): "mnAB"}[l]


def _mn(elem: str, X: np.ndarray) -> np.ndarray:
    return to_mn("mxfp4" if elem == "e2m1" else "mxfp8", X)


def run_mixed_layout(w: dict, la: int, lb: int) -> torch.Tensor:
    A = _mn(w["elemA"], w["A"]) if la else w["A"]
    B = _mn(w["elemB"], w["B"]) if lb else w["B"]
    d = _gpu.to_dev({"A": A, "B": B, "sA": w["sA"], "sB": w["sB"]})
    return dbs.gemm_mx_mixed(w["elemA"], w["elemB"], d["A"], d["sA"], d["B"], d["sB"], K=w["K"], la=la, lb=lb)


@pytest.mark.parametrize("lay", LAYS, ids=_lid)
@pytest.mark.parametrize("pair", E5M2_PAIRS, ids=_pid)
@pytest.mark.parametrize("shape", LAYOUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_e5m2_layouts_match_oracle(shape, pair, lay):
    """E5M2 pairs with MN-major operands (transposed 8-bit reads) against the
    oracle on the K-major codes."""
    M, N, K = shape
    _gpu.say(f"[mixed] {_pid(pair)} {_lid(lay)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 510 + M % 41, 610 + N % 43, *pair)
    D = run_mixed_layout(w, *lay)
    torch.cuda.synchronize()
    if M * N <= 1 << 23:
        _gpu.check_full("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(74, M, N, 4096)
        _gpu.check_sampled("mxfp8", w, D.contiguous(), em, en)


@pytest.mark.parametrize("pair", E5M2_PAIRS, ids=_pid)
def test_e5m2_layouts_agree_bitwise(pair):
    """All four layout combinations give the same bits."""
    _gpu.say(f"[mixed] {_pid(pair)} all layouts agree")
    w = synth.workload("mxfp8", 2944, 3008, 512, 93, 94, *pair)
    outs = [_gpu.d_bits(run_mixed_layout(w, la, lb)) for la, lb in [(0, 0), *LAYS]]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


F4_PAIRS = [("e4m3", "e2m1"), ("e2m1", "e4m3"), ("e5m2", "e2m1"), ("e2m1", "e5m2")]
# K % 256 == 0: the E2M1 operand stays packed in a ring of its own.  256 x 64
# tiles (K = 256: one 256-K stage per tile, so every load after the first
# crosses to the next tile; K = 1024 with several tiles per workgroup) and
# 256 x 256 tiles (chunked scales at K = 1024, per-stage scales at K = 768).
F4_SHAPES = [(300, 520, 256), (256, 20000, 1024), (3000, 2900, 1024), (2944, 3008, 768), (4100, 4200, 512)]


@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
@pytest.mark.parametrize("shape", F4_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_fp4_packed_matches_oracle(shape, pair):
    M, N, K = shape
    _gpu.say(f"[mixed] packed {_pid(pair)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 520 + M % 37, 620 + N % 31, *pair)
    D = run_mixed(w)
    torch.cuda.synchronize()
    if M * N <= 1 << 23:
        _gpu.check_full("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(75, M, N, 4096)
        _gpu.check_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
@pytest.mark.parametrize("mn", [(288, 320), (2944, 3008)], ids=lambda s: "x".join(map(str, s)))
def test_fp8_fp4_packed_unaligned_scales(pair, mn):
    """Scale rows whose base is not dword aligned: register-staged scales
    beside the packed E2M1 ring (256 x 64 tiles and the 4-wave 256 x 256)."""
    M, N = mn
    K = 512
    _gpu.say(f"[mixed] packed {_pid(pair)} unaligned scales {M}x{N}x{K}")
    w = synth.workload("mxfp8", M, N, K, 17, 18, *pair)
    d = _gpu.to_dev({"A": w["A"], "B": w["B"]})
    sa = torch.zeros(w["sA"].size + 1, dtype=torch.uint8, device="cuda")
    sb = torch.zeros(w["sB"].size + 1, dtype=torch.uint8, device="cuda")
    sa[1:] = torch.from_numpy(w["sA"].reshape(-1)).cuda()
    sb[1:] = torch.from_numpy(w["sB"].reshape(-1)).cuda()
    D = dbs.gemm_mx_mixed(pair[0], pair[1], d["A"], sa[1:].view(M, K // 32), d["B"], sb[1:].view(N, K // 32), K=K)
    torch.cuda.synchronize()
    _gpu.check_full("mxfp8", w, D)


@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
@pytest.mark.parametrize("mk", [(300, 1024), (3000, 2048)], ids=lambda s: "x".join(map(str, s)))
def test_fp8_fp4_packed_exact_permutation(pair, mk):
    """A times a permutation matrix with non-unit scales, bit for bit, on the
    packed E2M1 path."""
    M, K = mk
    ea, eb = pair
    _gpu.say(f"[mixed] packed {_pid(pair)} exact permutation {M}x{K}x{K}")
    rng = np.random.default_rng(41)
    N = K
    w = _pins.make_w_mx8(ea, eb, M, N, K, rng, scale_lo=110, scale_hi=140)
    pi = rng.permutation(K)
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), pi] = {"e5m2": 0x3C, "e4m3": 0x38, "e2m1": 0x2}[eb]
    if eb == "e2m1":
        B = (B[:, 0::2] | (B[:, 1::2] << 4)).astype(np.uint8)
    w["B"] = B
    w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    D = run_mixed(w)
    torch.cuda.synchronize()
    if M * K <= 1 << 20:
        _gpu.check_exact("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(42, M, N, 4096)
        _gpu.check_exact_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
def test_fp8_fp4_packed_random_codes(pair):
    """Codes over each format's whole finite range with random non-unit scales."""
    _gpu.say(f"[mixed] packed {_pid(pair)} random codes")
    w = _pins.make_w_mx8(*pair, 300, 280, 512, np.random.default_rng(29), scale_lo=112, scale_hi=142)
    D = run_mixed(w)
    torch.cuda.synchronize()
    _gpu.check_full("mxfp8", w, D)


# MN-major operands on the packed path (K % 256 == 0; M, N multiples of 32
# for whole 16-byte E2M1 K-rows): 256 x 64 tiles, 256 x 256 tiles with
# per-stage (K = 768) and chunked (K = 1024) scales
F4_LAYOUT_SHAPES = [(288, 320, 512), (256, 19968, 1024), (2944, 3072, 768), (3008, 2944, 1024)]


@pytest.mark.parametrize("lay", LAYS, ids=_lid)
@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
@pytest.mark.parametrize("shape", F4_LAYOUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_fp4_layouts_match_oracle(shape, pair, lay):
    M, N, K = shape
    _gpu.say(f"[mixed] packed {_pid(pair)} {_lid(lay)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 530 + M % 29, 630 + N % 23, *pair)
    D = run_mixed_layout(w, *lay)
    torch.cuda.synchronize()
    if M * N <= 1 << 23:
        _gpu.check_full("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(76, M, N, 4096)
        _gpu.check_sampled("mxfp8", w, D.contiguous(), em, en)


@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
def test_fp8_fp4_layouts_agree_bitwise(pair):
    """All four layout combinations of the packed path give the same bits."""
    _gpu.say(f"[mixed] packed {_pid(pair)} all layouts agree")
    w = synth.workload("mxfp8", 2944, 3008, 1024, 95, 96, *pair)
    outs = [_gpu.d_bits(run_mixed_layout(w, la, lb)) for la, lb in [(0, 0), *LAYS]]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("lay", LAYS, ids=_lid)
@pytest.mark.parametrize("pair", [("e4m3", "e2m1"), ("e2m1", "e5m2")], ids=_pid)
def test_fp8_fp4_layouts_unaligned_scales(pair, lay):
    """Register-staged scales (rows not dword aligned) with MN-major operands
    on the packed path (the 4-wave 256 x 256 tiles)."""
    M, N, K = 2944, 3008, 512
    _gpu.say(f"[mixed] packed {_pid(pair)} {_lid(lay)} unaligned scales")
    w = synth.workload("mxfp8", M, N, K, 19, 20, *pair)
    A = _mn(pair[0], w["A"]) if lay[0] else w["A"]
    B = _mn(pair[1], w["B"]) if lay[1] else w["B"]
    d = _gpu.to_dev({"A": A, "B": B})
    sa = torch.zeros(w["sA"].size + 1, dtype=torch.uint8, device="cuda")
    sb = torch.zeros(w["sB"].size + 1, dtype=torch.uint8, device="cuda")
    sa[1:] = torch.from_numpy(w["sA"].reshape(-1)).cuda()
    sb[1:] = torch.from_numpy(w["sB"].reshape(-1)).cuda()
    D = dbs.gemm_mx_mixed(pair[0], pair[1], d["A"], sa[1:].view(M, K // 32), d["B"], sb[1:].view(N, K // 32), K=K,
                          la=lay[0], lb=lay[1])
    torch.cuda.synchronize()
    em, en = synth.sample_entries(77, M, N, 4096)
    _gpu.check_sampled("mxfp8", w, D.contiguous(), em, en)


@pytest.mark.parametrize("pair", F4_PAIRS, ids=_pid)
def test_fp8_fp4_packed_edges(pair):
    """Single rows and columns on the packed path (K % 256 == 0): one output
    tile whose other rows read zero, and K of one 256-K stage."""
    for M, N, K in [(1, 1, 256), (1, 300, 512), (300, 1, 512), (2, 3, 256)]:
        _gpu.say(f"[mixed] packed {_pid(pair)} edge {(M, N, K)}")
        w = synth.workload("mxfp8", M, N, K, 43, 44, *pair)
        D = run_mixed(w)
        torch.cuda.synchronize()
        _gpu.check_full("mxfp8", w, D)


FP6_PAIRS = [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e3m2", "e4m3"), ("e4m3", "e2m3"),
             ("e5m2", "e3m2"), ("e2m3", "e5m2")]
# FP6: register-staged scales (K = 352), per-stage scales (K = 512), a
# square-ish problem (72 tiles of 256 x 64, one per workgroup)
FP6_SHAPES = [(300, 520, 352), (256, 4000, 512), (1000, 1100, 1024)]


@pytest.mark.parametrize("pair", FP6_PAIRS, ids=_pid)
@pytest.mark.parametrize("shape", FP6_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp6_matches_oracle(shape, pair):
    M, N, K = shape
    _gpu.say(f"[mixed] fp6 {_pid(pair)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 540 + M % 19, 640 + N % 17, *pair)
    D = run_mixed(w)
    torch.cuda.synchronize()
    _gpu.check_full("mxfp8", w, D)


@pytest.mark.parametrize("pair", FP6_PAIRS, ids=_pid)
def test_fp6_many_tiles_per_workgroup(pair):
    """More output tiles than CUs (1024 x 4160: 4 x 65 = 260 tiles of
    256 x 64), so workgroups run a second tile whose first stages were loaded
    during the first one's last."""
    M, N, K = 1024, 4160, 256
    _gpu.say(f"[mixed] fp6 {_pid(pair)} {M}x{N}x{K} (260 tiles)")
    w = synth.workload("mxfp8", M, N, K, 551, 651, *pair)
    D = run_mixed(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(78, M, N, 4096)
    _gpu.check_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("pair", [("e2m3", "e2m3"), ("e3m2", "e4m3")], ids=_pid)
def test_fp6_many_tiles_exact_permutation(pair):
    """A permutation B over 260 tiles of 256 x 64 with K = 4160 (a partial
    last 128-K stage), bit for bit on sampled entries."""
    ea, eb = pair
    M, K = 1024, 4160
    N = K
    _gpu.say(f"[mixed] fp6 {_pid(pair)} exact permutation {M}x{N}x{K}")
    rng = np.random.default_rng(53)
    w = _pins.make_w_mx8(ea, eb, M, N, K, rng, scale_lo=110, scale_hi=140)
    pi = rng.permutation(K)
    one = {"e5m2": 0x3C, "e4m3": 0x38, "e2m3": 0x08, "e3m2": 0x0C}[eb]
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), pi] = one
    w["B"] = synth.pack_fp6_rows(codes) if eb in ("e2m3", "e3m2") else codes
    w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    D = run_mixed(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(79, M, N, 4096)
    _gpu.check_exact_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("shape", [(1024, 4160, 384), (4352, 4096, 384)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("pair", [("e4m3", "e2m1"), ("e2m1", "e5m2")], ids=_pid)
def test_e2m1_widening_many_tiles_per_workgroup(shape, pair):
    """The E2M1 widening path (K % 256 == 128) with more tiles than CUs:
    260 tiles of 256 x 64 and 272 of 256 x 256."""
    M, N, K = shape
    _gpu.say(f"[mixed] widen {_pid(pair)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 552, 652, *pair)
    D = run_mixed(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(80, M, N, 4096)
    _gpu.check_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("pair", FP6_PAIRS, ids=_pid)
def test_fp6_random_codes(pair):
    """All 64 codes of each FP6 format with random non-unit scales."""
    _gpu.say(f"[mixed] fp6 {_pid(pair)} random codes")
    w = _pins.make_w_mx8(*pair, 300, 280, 256, np.random.default_rng(31), scale_lo=112, scale_hi=142)
    D = run_mixed(w)
    torch.cuda.synchronize()
    _gpu.check_full("mxfp8", w, D)


@pytest.mark.parametrize("pair", FP6_PAIRS, ids=_pid)
def test_fp6_exact_permutation(pair):
    """A times a permutation matrix in elem_b with non-unit scales, bit for bit:
    every output is one decoded FP6 (or 8-bit) element of A times two powers
    of two."""
    ea, eb = pair
    M, K = 300, 512
    N = K
    _gpu.say(f"[mixed] fp6 {_pid(pair)} exact permutation")
    rng = np.random.default_rng(47)
    w = _pins.make_w_mx8(ea, eb, M, N, K, rng, scale_lo=110, scale_hi=140)
    pi = rng.permutation(K)
    one = {"e5m2": 0x3C, "e4m3": 0x38, "e2m3": 0x08, "e3m2": 0x0C}[eb]
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), pi] = one
    w["B"] = synth.pack_fp6_rows(codes) if eb in ("e2m3", "e3m2") else codes
    w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    D = run_mixed(w)
    torch.cuda.synchronize()
    _gpu.check_exact("mxfp8", w, D)


def test_fp6_edges():
    """Single rows and columns, K of one block."""
    for (M, N, K), pair in [((1, 1, 32), ("e2m3", "e2m3")), ((1, 300, 64), ("e3m2", "e4m3")),
                            ((300, 1, 96), ("e4m3", "e3m2"))]:
        _gpu.say(f"[mixed] fp6 {_pid(pair)} edge {(M, N, K)}")
        w = synth.workload("mxfp8", M, N, K, 45, 46, *pair)
        D = run_mixed(w)
        torch.cuda.synchronize()
        _gpu.check_full("mxfp8", w, D)
