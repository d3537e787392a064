"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: bit-exact where the exact result is representable (identity,
permutation, power-of-two scale shifts, integer bf16); elsewhere
r = |D - D_ref| / (||dA_m|| ||dB_n|| |alpha|) <= 1e-2 and within the derived
bound 2^-8 + K 2^-23 of a correct fp32-accumulating path (tests/_gpu.py).
"""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu, _pins

pytestmark = pytest.mark.gpu

FMTS = ["bf16", "mxfp8", "mxfp4", "nvfp4"]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _w(fmt, M, N, K, seed=1):
    return synth.workload(fmt, M, N, K, 100 * seed + 1, 100 * seed + 2)


# ---- the small seeded config and ragged shapes, full comparison ----------------

@pytest.mark.parametrize("fmt", FMTS)
def test_cube_256(fmt):
    _gpu.say(f"[parity] {fmt} 256^3 seed 0")
    w = _w(fmt, 256, 256, 256, seed=0)
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    _gpu.check_full(fmt, w, D)


# The library picks 256 x 256 output tiles unless they would occupy at most
# half of the CUs, and 256 x 64 tiles otherwise.  RAGGED exercises the
# 256 x 64 path, SQUARE_RAGGED the 256 x 256 one (test_shape_lists_cover_both
# checks the split against the device's CU count).  MX rows of K/32 scale
# bytes that are not whole dwords (K % 128 != 0) take the register-staged
# scale path.
RAGGED = [
    (300, 520, 352),      # partial tiles in M and N, partial last K stage
    (257, 129, 96),       # one row / one column past a tile edge
    (1, 1, 32),           # single output
    (33, 7, 64),          # N not a multiple of 4 (element-wise stores)
    (512, 260, 4096),     # long K: many ring rotations
    (256, 20000, 512),    # 313 tiles: several per workgroup through the stage stream; MXFP4 has
                          # 2 stages per tile (the 3-slot ring's loads run a whole tile ahead)
    (300, 9000, 768),     # 282 tiles, ragged M and N; NVFP4 takes the 4-wave raw kernel (K % 256 == 0)
                          # with three stages per tile, streamed across a workgroup's tiles
]
SQUARE_RAGGED = [
    (3000, 2900, 352),    # partial tiles, partial last stage; MX scale rows of 11 bytes
    (2900, 3000, 384),    # MX scale rows of whole dwords
    (2100, 4200, 640),    # partial last MXFP4 stage (640 = 2.5 x 256)
    (5000, 4100, 96),     # 340 tiles > one persistent round
    (2600, 3000, 64),     # a single stage (BF16, NVFP4); MX scale rows of 2 bytes
]


def _square_tiles(M, N):
    return -(-M // 256) * -(-N // 256)


def test_shape_lists_cover_both():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert all(2 * _square_tiles(M, N) <= cus for M, N, _ in RAGGED)
    assert all(2 * _square_tiles(M, N) > cus for M, N, _ in SQUARE_RAGGED)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", RAGGED + SQUARE_RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged(fmt, shape):
    M, N, K = shape
    _gpu.say(f"[parity] {fmt} ragged {shape}")
    w = _w(fmt, M, N, K, seed=3)
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    _gpu.check_full(fmt, w, D)


@pytest.mark.parametrize("fmt", FMTS)
def test_random_codes_and_scales(fmt):
    """Codes over the whole finite range with random non-unit scales at small K,
    where one mis-applied block scale would give r >> 1e-2."""
    _gpu.say(f"[parity] {fmt} random codes K=64")
    rng = np.random.default_rng(21)
    kw = {"scale_lo": 112, "scale_hi": 142}
    if fmt == "nvfp4":
        kw = {"scale_lo": 0x08, "scale_hi": 0x7E}
    if fmt == "bf16":
        kw = {"bf16_exp": (110, 144)}
    w = _pins.make_w(fmt, 300, 280, 64, rng, **kw)
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    _gpu.check_full(fmt, w, D)


@pytest.mark.parametrize("shape", [(300, 3000, 512), (3000, 2900, 768)], ids=lambda s: "x".join(map(str, s)))
def test_nvfp4_random_codes_and_scales_raw(shape):
    """NVFP4 codes over the whole E2M1 range with random E4M3 scales (most of
    the finite range) through the raw-staged kernels' pipelined decode:
    4-wave 256 x 64 tiles and 8-wave 256 x 256 tiles, several stages."""
    M, N, K = shape
    _gpu.say(f"[parity] nvfp4 random codes and scales {shape}")
    rng = np.random.default_rng(23)
    w = _pins.make_w("nvfp4", M, N, K, rng, scale_lo=0x08, scale_hi=0x7E)
    D = _gpu.run("nvfp4", w)
    torch.cuda.synchronize()
    if M * N <= 1_000_000:
        _gpu.check_full("nvfp4", w, D)
    else:
        em, en = synth.sample_entries(24, M, N, 4096)
        _gpu.check_sampled("nvfp4", w, D, em, en)


# ---- bit-exact cases ------------------------------------------------------------

def _identity_w(fmt, M, K, rng, permute):
    N = K
    pi = rng.permutation(K) if permute else np.arange(K)
    kw = {"scale_lo": 110, "scale_hi": 140} if fmt != "nvfp4" else {"scale_lo": 0x10, "scale_hi": 0x70}
    a = _pins.random_codes(fmt, M, K, rng, **kw)
    w = {"fmt": fmt, "M": M, "N": N, "K": K, "A": a["X"]}
    if fmt == "bf16":
        B = np.zeros((N, K), np.uint16)
        B[np.arange(N), pi] = 0x3F80
    elif fmt == "mxfp8":
        B = np.zeros((N, K), np.uint8)
        B[np.arange(N), pi] = 0x38
    else:
        codes = np.zeros((N, K), np.uint8)
        codes[np.arange(N), pi] = 0x2
        B = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w["B"] = B
    if fmt in ("mxfp8", "mxfp4"):
        w["sA"] = a["s"]
        w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    elif fmt == "nvfp4":
        w["sA"] = a["s"]
        w["sB"] = rng.integers(0x28, 0x50, (N, K // 16)).astype(np.uint8)   # non-power-of-two E4M3
        w["tA"], w["tB"] = 1.0, 1.0
    return w


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("permute", [False, True], ids=["identity", "permutation"])
def test_exact_identity_permutation(fmt, permute):
    _gpu.say(f"[exact] {fmt} permute={permute}")
    rng = np.random.default_rng(31)
    w = _identity_w(fmt, 300, 512, rng, permute)
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    _gpu.check_exact(fmt, w, D)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mk", [(3000, 2944), (4100, 4608)], ids=lambda s: "x".join(map(str, s)))
def test_exact_permutation_square_tiles(fmt, mk):
    """The permutation test at shapes that take 256 x 256 tiles, checked bit
    for bit on sampled entries.  4100 x 4608 x 4608: 306 tiles (some
    workgroups take two), and K = 4608 gives MXFP8 36 and MXFP4 18 stages per
    tile, whole chunks of stage scales (4 and 2 stages)."""
    M, K = mk
    _gpu.say(f"[exact] {fmt} permutation {M}x{K}x{K}")
    rng = np.random.default_rng(33)
    w = _identity_w(fmt, M, K, rng, True)
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(34, w["M"], w["N"], 4096)
    _gpu.check_exact_sampled(fmt, w, D, em, en)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("shape", [(260, 300, 512), (3000, 2900, 512), (256, 20000, 768)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_pow2_scale_shift(fmt, shape):
    """Moving every A scale by a power of two (E8M0 code +3; E4M3 exponent
    field -3) scales every output by exactly that power."""
    _gpu.say(f"[exact] {fmt} pow2 shift {shape}")
    w = _w(fmt, *shape, seed=4)
    D0 = _gpu.d_bits(_gpu.run(fmt, w))
    w2 = dict(w)
    if fmt == "nvfp4":
        assert w["sA"].min() >= 0x20          # stays a normal E4M3 value
        w2["sA"] = (w["sA"].astype(np.int64) - 24).astype(np.uint8)
        factor = np.float32(0.125)
    else:
        w2["sA"] = (w["sA"].astype(np.int64) + 3).astype(np.uint8)
        factor = np.float32(8.0)
    D1 = _gpu.d_bits(_gpu.run(fmt, w2))
    torch.cuda.synchronize()
    f0 = (D0.astype(np.uint32) << 16).view(np.float32)
    f1 = (D1.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f1, f0 * factor)


@pytest.mark.parametrize("shape", [(300, 270, 1024), (3000, 2900, 256)], ids=lambda s: "x".join(map(str, s)))
def test_exact_bf16_integers(shape):
    """bf16 integer inputs in [-8, 8] at K <= 1024: every partial sum is an
    integer below 2^24, so the fp32 result is exact and so is bf16(D)."""
    _gpu.say(f"[exact] bf16 integers {shape}")
    rng = np.random.default_rng(41)
    M, N, K = shape
    ia = rng.integers(-8, 9, (M, K)).astype(np.float32)
    ib = rng.integers(-8, 9, (N, K)).astype(np.float32)
    w = {"fmt": "bf16", "M": M, "N": N, "K": K,
         "A": (ia.view(np.uint32) >> 16).astype(np.uint16), "B": (ib.view(np.uint32) >> 16).astype(np.uint16)}
    D = _gpu.run("bf16", w)
    torch.cuda.synchronize()
    _gpu.check_exact("bf16", w, D)


@pytest.mark.parametrize("shape", [(300, 520, 80), (257, 129, 16), (33, 7, 48), (256, 20000, 336),
                                   (3000, 2900, 208)], ids=lambda s: "x".join(map(str, s)))
def test_nvfp4_k_odd_multiple_of_16(shape):
    """K an odd multiple of 16, which the NVFP4 format allows: packed rows
    start on 8-byte and scale rows on byte boundaries, and each row ends with
    one 16-element block of a 32-element half-row (256 x 64 and 256 x 256
    tiles)."""
    M, N, K = shape
    _gpu.say(f"[parity] nvfp4 K % 32 == 16 {shape}")
    w = _w("nvfp4", M, N, K, seed=9)
    D = _gpu.run("nvfp4", w)
    torch.cuda.synchronize()
    _gpu.check_full("nvfp4", w, D)


@pytest.mark.parametrize("mk", [(300, 208), (3000, 2960)], ids=lambda s: "x".join(map(str, s)))
def test_exact_nvfp4_k_odd_multiple_of_16(mk):
    """The permutation test with K an odd multiple of 16, bit for bit."""
    M, K = mk
    _gpu.say(f"[exact] nvfp4 permutation {M}x{K}x{K}")
    w = _identity_w("nvfp4", M, K, np.random.default_rng(37), True)
    D = _gpu.run("nvfp4", w)
    torch.cuda.synchronize()
    if M * K <= 1 << 20:
        _gpu.check_exact("nvfp4", w, D)
    else:
        em, en = synth.sample_entries(38, M, K, 4096)
        _gpu.check_exact_sampled("nvfp4", w, D, em, en)


def test_exact_nvfp4_tensor_scales():
    """NVFP4 with power-of-two tensor scales tA = 2, tB = 0.25 on an identity B."""
    _gpu.say("[exact] nvfp4 tensor scales")
    rng = np.random.default_rng(51)
    w = _identity_w("nvfp4", 64, 256, rng, True)
    w["tA"], w["tB"] = 2.0, 0.25
    D = _gpu.run("nvfp4", w)
    torch.cuda.synchronize()
    _gpu.check_exact("nvfp4", w, D)


@pytest.mark.parametrize("K", [256, 512, 768])
@pytest.mark.parametrize("shift", [0, 4, 1], ids=["scales16", "scales4", "scales1"])
def test_nvfp4_skinny_kernel_choice(K, shift):
    """K-major NVFP4 on 256 x 64 tiles through each kernel the launcher picks:
    the 4-wave raw kernel (16-byte-aligned scale rows, K % 256 == 0, two or
    more stages), and the kernels that decode into LDS (a single stage, scale
    rows on 4-byte or 1-byte boundaries)."""
    M, N = 300, 3000
    _gpu.say(f"[parity] nvfp4 skinny K={K} scale offset {shift}")
    w = _w("nvfp4", M, N, K, seed=13)
    d = _gpu.to_dev(w)
    sa = torch.zeros(w["sA"].size + 16, dtype=torch.uint8, device="cuda")
    sb = torch.zeros(w["sB"].size + 16, dtype=torch.uint8, device="cuda")
    sa[shift:shift + w["sA"].size] = torch.from_numpy(w["sA"].reshape(-1)).cuda()
    sb[shift:shift + w["sB"].size] = torch.from_numpy(w["sB"].reshape(-1)).cuda()
    D = dbs.gemm_nvfp4(d["A"], sa[shift:shift + w["sA"].size].view(M, K // 16), w["tA"],
                       d["B"], sb[shift:shift + w["sB"].size].view(N, K // 16), w["tB"])
    torch.cuda.synchronize()
    _gpu.check_full("nvfp4", w, D)


# ---- determinism (a race canary) ---------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_repeat_bit_identical(fmt):
    _gpu.say(f"[determinism] {fmt}")
    w = _w(fmt, 1024, 768, 1024, seed=5)
    dev = _gpu.to_dev(w)
    first = _gpu.run(fmt, w, dev).view(torch.int16).clone()
    again = torch.empty_like(first).view(torch.bfloat16)
    for i in range(100):
        _gpu.run(fmt, w, dev, out=again)
        assert torch.equal(first, again.view(torch.int16)), f"repeat {i} differs"


def test_out_argument_and_stream():
    """Writing into a caller-provided output on a non-default stream."""
    _gpu.say("[abi] out= on a side stream")
    w = _w("bf16", 256, 256, 256, seed=6)
    dev = _gpu.to_dev(w)
    out = torch.full((256, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _gpu.run("bf16", w, dev, out=out)
    s.synchronize()
    _gpu.check_full("bf16", w, out)
