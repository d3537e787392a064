"""CPU pins of the oracle's NVFP4 -> MXFP8 requantisation (the opt-in
FP8-rate NVFP4 GEMM), against an independent derivation: values from the
OCP E2M1 table and torch's float8 decoders, rounding by torch's cast to
float8_e4m3fn (round to nearest even)."""
import numpy as np
import torch

import oracle
from tests import _pins


def _nvfp4_operand(rng, rows, K, scale_lo=0x08, scale_hi=0x7E):
    codes = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (rows, K // 16)).astype(np.uint8)
    return codes, scales


def _independent(codes, scales, K):
    """Requantised codes and E8M0 scales, derived with numpy / torch only."""
    rows = codes.shape[0]
    el = np.empty((rows, K), np.uint8)
    el[:, 0::2] = codes & 0xF
    el[:, 1::2] = codes >> 4
    a = _pins.ref_e2m1(el)                                       # (rows, K) values
    s = _pins.ref_e4m3(scales)                                   # (rows, K/16)
    s32 = np.maximum(np.abs(s[:, 0::2]), np.abs(s[:, 1::2]))    # per 32-block
    _, ex = np.frexp(s32)
    E = np.where(s32 > 0, ex - 1, 0)
    v = a * np.repeat(s, 16, axis=1) * np.repeat(np.ldexp(1.0, -E), 32, axis=1)
    q = torch.from_numpy(v).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, (E + 127).astype(np.uint8), a * np.repeat(s, 16, axis=1), E


def test_requant_matches_independent_derivation():
    rng = np.random.default_rng(81)
    K = 256
    codes, scales = _nvfp4_operand(rng, 64, K)
    scales[0, :] = 0                                             # zero groups
    scales[1, 0::2] = 0                                          # one zero group per block
    scales[2, :] = 0x01                                          # smallest subnormal scale
    scales[3, :] = 0x7E                                          # 448
    out, osc = oracle.requant_nvfp4_mx8(codes, scales, K)
    q, e8, _, _ = _independent(codes, scales, K)
    assert np.array_equal(osc, e8)
    assert np.array_equal(out, q)


def test_requant_is_exact_at_unit_scales():
    """With unit E4M3 scales every E2M1 value is an E4M3 value: lossless."""
    rng = np.random.default_rng(82)
    K = 128
    codes, _ = _nvfp4_operand(rng, 16, K)
    scales = np.full((16, K // 16), 0x38, np.uint8)              # 1.0
    out, osc = oracle.requant_nvfp4_mx8(codes, scales, K)
    assert np.all(osc == 127)
    _, _, exact, _ = _independent(codes, scales, K)
    assert np.array_equal(oracle.decode("e4m3", out), exact)


def test_requant_error_bound():
    """Per element: |requantised - exact| <= 2^-4 |exact| where the scaled
    value is an E4M3 normal (>= 2^-6), else <= 2^-10 * 2^E (half the
    subnormal step), with 2^E <= max(s0, s1) < 2^(E+1)."""
    rng = np.random.default_rng(83)
    K = 512
    codes, scales = _nvfp4_operand(rng, 128, K)
    out, osc = oracle.requant_nvfp4_mx8(codes, scales, K)
    _, _, exact, E = _independent(codes, scales, K)
    got = oracle.decode("e4m3", out) * np.repeat(np.ldexp(1.0, E), 32, axis=1)
    err = np.abs(got - exact)
    scaled = np.abs(exact) * np.repeat(np.ldexp(1.0, -E), 32, axis=1)
    normal = scaled >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(exact[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * np.repeat(np.ldexp(1.0, E), 32, axis=1)[~normal])
    assert np.all(np.abs(oracle.decode("e4m3", out)) < 12.0)      # never near E4M3's 448
