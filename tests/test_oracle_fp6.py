"""Pins of the oracle's FP6 element formats (E2M3, E3M2) and their packing.

The OCP MX v1.0 anchor values (tests/golden/ocp_fp6_anchors.txt), torch's
independent E4M3 / E5M2 conversions (every E2M3 value is an E4M3 value, every
E3M2 value an E5M2 value), round trips over all 64 codes, a hand-checked
packing fixture, the input generator's independent packing and quantiser,
and planted mistakes that each of these catches."""
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = Path(__file__).parent / "golden" / "ocp_fp6_anchors.txt"


def _anchors():
    rows = []
    for line in GOLDEN.read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            f, c, v = line.split()
            rows.append((f, int(c, 16), float(v)))
    return rows


def _anchors_hold():
    for f, c, v in _anchors():
        got = float(oracle.decode(f, np.array([c], np.uint8))[0])
        if got != v or np.signbit(got) != np.signbit(v):
            return False
    return True


def test_anchor_values():
    assert _anchors_hold()


@pytest.mark.parametrize("fmt,f8", [("e2m3", torch.float8_e4m3fn), ("e3m2", torch.float8_e5m2)])
def test_values_are_exact_in_the_wider_8bit_format(fmt, f8):
    """torch's own conversion to the 8-bit format leaves every value unchanged
    (the widening the FP6 GEMM path relies on is exact)."""
    v = oracle.decode(fmt, np.arange(64, dtype=np.uint8))
    t = torch.from_numpy(v).to(torch.float32)
    assert torch.equal(t.to(f8).to(torch.float32), t)


@pytest.mark.parametrize("fmt,nmax", [("e2m3", 7.5), ("e3m2", 28.0)])
def test_codes_round_trip_and_order(fmt, nmax):
    c = np.arange(64, dtype=np.uint8)
    v = oracle.decode(fmt, c)
    assert np.array_equal(oracle.encode(fmt, v), c)
    pos = v[:32]
    assert np.all(np.diff(pos) > 0) and pos[-1] == nmax
    assert np.array_equal(v[32:], -pos)
    # beyond the largest value: saturation
    assert oracle.encode(fmt, np.array([1e9, -1e9])).tolist() == [0x1F, 0x3F]


def test_packing_fixture():
    """Element j of a row at bits 6j .. 6j+5 of its little-endian bytes."""
    packed = np.array([[0x01, 0x00, 0x00, 0x40, 0x00, 0x00, 0x00, 0x00, 0x80, 0xFF, 0x0F, 0x00]], np.uint8)
    codes = oracle.unpack_fp6(packed, 16)
    assert codes[0].tolist() == [1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 0, 0x20, 0x3F, 0x3F, 0, 0]
    assert np.array_equal(synth.unpack_fp6_rows(packed, 16), codes)


def test_packing_agrees_with_generator():
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (5, 48), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_fp6(packed, 64), synth.unpack_fp6_rows(packed, 64))
    codes = rng.integers(0, 64, (5, 64), dtype=np.uint8)
    assert np.array_equal(synth.unpack_fp6_rows(synth.pack_fp6_rows(codes), 64), codes)


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_quantiser_agrees_with_generator(elem):
    x = synth.normal(11, 23, 320)
    c1, s1 = synth.quant_mx(x, elem)
    c2, s2 = oracle.quant_mx(x, elem)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_gemm_reads_fp6_elements():
    """A one-hot FP6 B row picks one element of A, times the two scales."""
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 64
    for ea in ("e2m3", "e3m2"):
        a_codes = rng.integers(0, 64, (M, K), dtype=np.uint8)
        pi = rng.permutation(K)[:N]
        b_codes = np.zeros((N, K), np.uint8)
        b_codes[np.arange(N), pi] = {"e2m3": 0x08, "e3m2": 0x0C}[ea]          # 1.0
        sA = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
        sB = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
        w = {"fmt": "mxfp8", "M": M, "N": N, "K": K, "elemA": ea, "elemB": ea,
             "A": synth.pack_fp6_rows(a_codes), "sA": sA, "B": synth.pack_fp6_rows(b_codes), "sB": sB}
        d, _, _ = oracle.gemm_full("mxfp8", w, nthreads=1)
        va = oracle.decode(ea, a_codes)
        for n in range(N):
            k = pi[n]
            want = va[:, k] * 2.0 ** (sA[:, k // 32].astype(int) - 127) * 2.0 ** (int(sB[n, k // 32]) - 127)
            assert np.array_equal(d[:, n], want)


@pytest.mark.parametrize("mut,check", [
    (14, _anchors_hold),                        # E2M3 bias 2
    (15, _anchors_hold),                        # E3M2 subnormals as normals
    (16, lambda: oracle.unpack_fp6(np.array([[0x01, 0x00, 0x00]], np.uint8), 4)[0].tolist() == [1, 0, 0, 0]),
])
def test_planted_mistakes_are_caught(mut, check):
    lib = oracle._load()
    lib.orc_set_mutation(mut)
    try:
        assert not check()
    finally:
        lib.orc_set_mutation(0)
