"""GPU parity of the native-rate FP6 path (FP6 on both operands; 256 x 256
tiles; K a multiple of 128; scales per stage, or in chunks of four stages
when K % 512 == 0): every E2M3 / E3M2 pairing against the oracle,
codes over all 64 values with random scales, exact permutation products with
non-unit scales, ragged edges, a second persistent round, and the smallest K
the three-slot ring takes.  Smaller FP6 problems take the widening path
(test_gpu_mixed.py)."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu, _pins

pytestmark = pytest.mark.gpu

PAIRS = [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e3m2", "e2m3")]
ONE = {"e2m3": 0x08, "e3m2": 0x0C}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _pid(p):
    return f"{p[0]}x{p[1]}"


def run(w: dict) -> torch.Tensor:
    d = _gpu.to_dev(w)
    return dbs.gemm_mx_mixed(w["elemA"], w["elemB"], d["A"], d["sA"], d["B"], d["sB"], K=w["K"])


def check(w, D, seed):
    M, N = w["M"], w["N"]
    if M * N <= 6 << 20:
        _gpu.check_full("mxfp8", w, D)
    else:
        em, en = synth.sample_entries(seed, M, N, 4096)
        _gpu.check_sampled("mxfp8", w, D, em, en)


# Per-stage scales (K % 512 != 0): ragged 9 x 10 tiles with K of three
# stages (the ring wraps inside a tile); 289 tiles (a second persistent
# round) with K of two stages, the smallest the ring takes.  Chunked scales
# (four stages a chunk): 81 tiles with two chunks; 289 tiles with one chunk
# (every chunk load fetches the next tile's); 289 tiles with three chunks
# (the chunk buffers alternate across tiles); ragged tiles with four chunks.
SHAPES = [(2200, 2500, 384), (4352, 4352, 256), (2304, 2304, 1024), (4352, 4352, 512), (4352, 4352, 1536),
          (2200, 2500, 2048)]


@pytest.mark.parametrize("pair", PAIRS, ids=_pid)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp6_native_matches_oracle(shape, pair):
    M, N, K = shape
    _gpu.say(f"[fp6] {_pid(pair)} {shape}")
    w = synth.workload("mxfp8", M, N, K, 700 + M % 23, 800 + N % 29, *pair)
    D = run(w)
    torch.cuda.synchronize()
    check(w, D, 81)


@pytest.mark.parametrize("pair", PAIRS, ids=_pid)
def test_fp6_native_random_codes(pair):
    """All 64 codes of each format with random non-unit scales."""
    _gpu.say(f"[fp6] {_pid(pair)} random codes")
    w = _pins.make_w_mx8(*pair, 2304, 2048, 512, np.random.default_rng(57), scale_lo=112, scale_hi=142)
    D = run(w)
    torch.cuda.synchronize()
    _gpu.check_full("mxfp8", w, D)


@pytest.mark.parametrize("K", [2304, 2048], ids=["per-stage-scales", "chunked-scales"])
@pytest.mark.parametrize("pair", PAIRS, ids=_pid)
def test_fp6_native_exact_permutation(pair, K):
    """A (random codes, random scales) times a permutation matrix in B's
    format with non-unit scales: every output is one element of A times two
    powers of two, compared bit for bit (sampled)."""
    ea, eb = pair
    M = 2304
    N = K
    _gpu.say(f"[fp6] {_pid(pair)} exact permutation {M}x{N}x{K}")
    rng = np.random.default_rng(59)
    w = _pins.make_w_mx8(ea, eb, M, N, K, rng, scale_lo=110, scale_hi=140)
    pi = rng.permutation(K)
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), pi] = ONE[eb]
    w["B"] = synth.pack_fp6_rows(codes)
    w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    D = run(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(82, M, N, 4096)
    _gpu.check_exact_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("K", [2304, 2048], ids=["per-stage-scales", "chunked-scales"])
def test_fp6_native_unit_scale_identity(K):
    """B = the identity (N = K) with unit scales: D reproduces A's decoded
    values exactly, so every fragment, unit rotation and ring slot lands
    where the MFMA expects it."""
    M = 2304
    _gpu.say(f"[fp6] identity K={K}")
    rng = np.random.default_rng(61)
    w = _pins.make_w_mx8("e2m3", "e2m3", M, K, K, rng, scale_lo=127, scale_hi=127)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = ONE["e2m3"]
    w["B"] = synth.pack_fp6_rows(codes)
    D = run(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(83, M, K, 4096)
    _gpu.check_exact_sampled("mxfp8", w, D, em, en)


@pytest.mark.parametrize("K", [256, 512], ids=["per-stage-scales", "chunked-scales"])
def test_fp6_native_layouts_of_d(K):
    """Output rows whose length is not a multiple of 8 take the direct
    stores instead of the staged epilogue."""
    M, N = 2304, 2300
    _gpu.say(f"[fp6] direct-store epilogue {M}x{N}x{K}")
    w = synth.workload("mxfp8", M, N, K, 711, 811, "e3m2", "e2m3")
    D = run(w)
    torch.cuda.synchronize()
    check(w, D, 84)


def test_fp6_native_chunks_across_rounds_exact():
    """Chunked scales over 324 tiles (a second persistent round) with nine
    chunks a tile (an odd count: the chunk buffers alternate across tiles): a
    permutation product with non-unit scales, bit for bit."""
    M, K = 4608, 4608
    N = K
    _gpu.say(f"[fp6] chunked exact permutation {M}x{N}x{K}")
    rng = np.random.default_rng(63)
    w = _pins.make_w_mx8("e2m3", "e3m2", M, N, K, rng, scale_lo=112, scale_hi=142)
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), rng.permutation(K)] = ONE["e3m2"]
    w["B"] = synth.pack_fp6_rows(codes)
    w["sB"] = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    D = run(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(88, M, N, 4096)
    _gpu.check_exact_sampled("mxfp8", w, D, em, en)
