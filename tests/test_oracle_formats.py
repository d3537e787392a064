"""CPU pins of the oracle's format codecs (OCP MX v1.0 element/scale types)."""
import math

import numpy as np
import pytest

import oracle
from tests import _pins


def test_decoders_match_independent_sources():
    assert _pins.check_decoders()


@pytest.mark.parametrize("name,fmt", [("ocp_e4m3_anchors.txt", "e4m3"), ("ocp_e8m0_anchors.txt", "e8m0"),
                                      ("ocp_e2m1.txt", "e2m1"), ("ocp_e5m2_anchors.txt", "e5m2")])
def test_anchor_tables(name, fmt):
    table = _pins._table(name)
    codes = np.array(sorted(table), np.uint8)
    got = oracle.decode(fmt, codes)
    for c, g in zip(codes, got):
        e = table[int(c)]
        if math.isnan(e):
            assert math.isnan(g)
        else:
            assert g == e and math.copysign(1, g) == math.copysign(1, e), (hex(c), g, e)


@pytest.mark.parametrize("fmt,ncodes,nan_codes", [("e2m1", 16, ()), ("e4m3", 256, (0x7F, 0xFF)),
                                                  ("e5m2", 256, tuple(range(0x7C, 0x80)) + tuple(range(0xFC, 0x100)))])
def test_encode_decode_round_trip(fmt, ncodes, nan_codes):
    codes = np.array([c for c in range(ncodes) if c not in nan_codes], np.uint8)
    vals = oracle.decode(fmt, codes)
    back = oracle.encode(fmt, vals)
    assert np.array_equal(back, codes)


def test_e2m1_ties_to_even():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -0.0, -4.0])
    got = oracle.decode("e2m1", oracle.encode("e2m1", x))
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))


def test_e4m3_ties_to_even_on_every_midpoint():
    codes = np.arange(0, 0x7E, dtype=np.uint8)          # consecutive finite positives
    lo = oracle.decode("e4m3", codes)
    hi = oracle.decode("e4m3", codes + 1)
    mid = (lo + hi) / 2                                   # exact in fp64
    got = oracle.encode("e4m3", mid)
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, even)


def test_saturation_and_signed_zero():
    assert oracle.encode("e4m3", np.array([1e9, 464.0, 470.0, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.encode("e2m1", np.array([7.0, 100.0, -100.0])).tolist() == [0x7, 0x7, 0xF]
    assert oracle.encode("e4m3", np.array([-0.0, 0.0, -1e-30])).tolist() == [0x80, 0x00, 0x80]
    assert oracle.encode("e2m1", np.array([-0.0, -0.2])).tolist() == [0x8, 0x8]


def test_bf16_encoder_matches_numpy_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # and the bottom of the range: fp32 subnormals (some round to the
    # smallest bf16 subnormal, some to +-0), signed zeros, the smallest normals
    tiny = np.array([1e-40, -3e-41, 1.4e-45, -1.4e-45, 2.0 ** -134, 2.0 ** -134 * 1.5, 2.0 ** -133,
                     -2.0 ** -133 * 0.75, 1.1754944e-38, 1e-38, 0.0, -0.0], np.float32)
    x = np.concatenate([x, tiny, -tiny, rng.standard_normal(4000).astype(np.float32) * np.float32(1e-39)])
    # numpy reference: fp32 -> bf16 RNE via integer rounding of the bit pattern
    b = x.view(np.uint32).astype(np.uint64)
    ref = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    got = oracle.encode("bf16", x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_nan_codes_decode_to_nan():
    assert np.isnan(oracle.decode("e4m3", np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.isnan(oracle.decode("e8m0", np.array([0xFF], np.uint8))).all()


def test_e5m2_ties_to_even_and_saturation():
    codes = np.arange(0, 0x7B, dtype=np.uint8)          # consecutive finite positives
    mid = (oracle.decode("e5m2", codes) + oracle.decode("e5m2", codes + 1)) / 2
    assert np.array_equal(oracle.encode("e5m2", mid), np.where(codes % 2 == 0, codes, codes + 1))
    assert oracle.encode("e5m2", np.array([1e9, 61440.0, -1e9, -0.0])).tolist() == [0x7B, 0x7B, 0xFB, 0x80]
