"""CPU pins of the oracle's NVFP4 -> MXFP8 and NVFP4 -> MXFP6 (E2M3)
requantisations (the opt-in FP8- and FP4-rate NVFP4 GEMMs), against an independent derivation: values from the
OCP E2M1 table and torch's float8 decoders, rounding by torch's cast to
float8_e4m3fn (round to nearest even)."""
import numpy as np
import torch

import oracle
import synth
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


# ---- NVFP4 -> MXFP6 (E2M3), the FP4-rate path -------------------------------------

def _nearest_e2m3(v):
    """Nearest E2M3 code of each value over the decoded code set (pinned to
    the OCP anchors in test_oracle_fp6), ties to the even code."""
    grid = oracle.decode("e2m3", np.arange(32, dtype=np.uint8))         # 0 .. 7.5, ascending
    a = np.abs(v)
    i = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 31)
    j = np.minimum(i + 1, 31)
    lo, hi = a - grid[i], grid[j] - a
    mag = np.where(lo < hi, i, np.where(hi < lo, j, np.where(i % 2 == 0, i, j)))
    mag = np.where(a >= grid[-1], 31, mag)
    return (mag | np.where(np.signbit(v), 32, 0)).astype(np.uint8)


def _independent_e2m3(codes, scales, K):
    """E2M3 codes and E8M0 scales by the stated rule: E the smallest integer
    with 6 m <= 7.5 * 2^E (m the block's larger |scale|), then the nearest
    code of a * s_g * 2^-E; derived with numpy / torch decoders only."""
    rows = codes.shape[0]
    el = np.empty((rows, K), np.uint8)
    el[:, 0::2] = codes & 0xF
    el[:, 1::2] = codes >> 4
    a = _pins.ref_e2m1(el)
    s = _pins.ref_e4m3(scales)
    m = np.maximum(np.abs(s[:, 0::2]), np.abs(s[:, 1::2]))
    E = np.zeros(m.shape, np.int64)
    nz = m > 0
    E[nz] = np.ceil(np.log2(6.0 * m[nz] / 7.5)).astype(np.int64)
    # the smallest such E, checked exactly (6 m and 7.5 * 2^E are exact doubles)
    assert np.all(6.0 * m[nz] <= 7.5 * np.ldexp(1.0, E[nz]))
    assert np.all(6.0 * m[nz] > 7.5 * np.ldexp(1.0, E[nz] - 1))
    exact = a * np.repeat(s, 16, axis=1)
    v = exact * np.repeat(np.ldexp(1.0, -E), 32, axis=1)
    return _nearest_e2m3(v), (E + 127).astype(np.uint8), exact, E, v


def test_e2m3_requant_matches_independent_derivation():
    rng = np.random.default_rng(84)
    K = 256
    codes, scales = _nvfp4_operand(rng, 64, K)
    scales[0, :] = 0
    scales[1, 0::2] = 0
    scales[2, :] = 0x01
    scales[3, :] = 0x7E
    scales[4, :] = 0x3A                                          # 1.25: the rule's boundary
    out, osc = oracle.requant_nvfp4_e2m3(codes, scales, K)
    q, e8, _, _, _ = _independent_e2m3(codes, scales, K)
    assert np.array_equal(osc, e8)
    assert np.array_equal(synth.unpack_fp6_rows(out, K), q)


def test_e2m3_requant_is_exact_at_unit_scales():
    rng = np.random.default_rng(85)
    K = 128
    codes, _ = _nvfp4_operand(rng, 16, K)
    scales = np.full((16, K // 16), 0x38, np.uint8)
    out, osc = oracle.requant_nvfp4_e2m3(codes, scales, K)
    assert np.all(osc == 127)
    _, _, exact, _, _ = _independent_e2m3(codes, scales, K)
    assert np.array_equal(oracle.decode("e2m3", synth.unpack_fp6_rows(out, K)), exact)


def test_e2m3_requant_error_bound():
    """Per element: |requantised - exact| <= max(2^-4 |exact|, 2^-4 * 2^E):
    E2M3 has three mantissa bits (half a step is 2^-4 relative) and a
    subnormal step of 1/8 below 1; the scaled values stay within 7.5."""
    rng = np.random.default_rng(86)
    K = 512
    codes, scales = _nvfp4_operand(rng, 128, K)
    out, osc = oracle.requant_nvfp4_e2m3(codes, scales, K)
    _, _, exact, E, v = _independent_e2m3(codes, scales, K)
    p2 = np.repeat(np.ldexp(1.0, E), 32, axis=1)
    got = oracle.decode("e2m3", synth.unpack_fp6_rows(out, K)) * p2
    assert np.all(np.abs(v) <= 7.5)
    assert np.all(np.abs(got - exact) <= np.maximum(2.0 ** -4 * np.abs(exact), 2.0 ** -4 * p2))


def test_e2m3_requant_planted_exponent_rule_is_caught():
    rng = np.random.default_rng(87)
    K = 128
    codes, scales = _nvfp4_operand(rng, 32, K)
    _, e8, _, _, _ = _independent_e2m3(codes, scales, K)
    oracle.set_mutation(20)
    try:
        _, osc = oracle.requant_nvfp4_e2m3(codes, scales, K)
    finally:
        oracle.set_mutation(0)
    assert not np.array_equal(osc, e8)
