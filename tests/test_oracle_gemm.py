"""CPU pins of the oracle GEMM: exact rationals, identity/permutation,
power-of-two scale shifts, textbook reductions, invariants."""
import numpy as np
import pytest

import oracle
from tests import _pins

FMTS = ["bf16", "mxfp8", "mxfp4", "nvfp4"]


@pytest.mark.parametrize("fmt", FMTS)
def test_fraction_brute_force(fmt):
    assert _pins.check_brute_force_fraction(fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_fraction_brute_force_exact_scales(fmt):
    assert _pins.check_brute_force_fraction(fmt, seed=10, exact_scales=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_identity(fmt):
    assert _pins.check_identity(fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_permutation_crossing_blocks(fmt):
    assert _pins.check_permutation(fmt)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_pow2_scale_shift(fmt):
    assert _pins.check_pow2_scale_shift(fmt)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_unit_scales_reduce_to_plain_matmul(fmt):
    assert _pins.check_unit_scale_matmul(fmt)


def test_bf16_integer_inputs_exact():
    assert _pins.check_bf16_integers()


def test_bf16_rectangular():
    assert _pins.check_rectangular_bf16()


@pytest.mark.parametrize("fmt", FMTS)
def test_transpose_symmetry(fmt):
    assert _pins.check_transpose_symmetry(fmt)


def test_nvfp4_alpha_linearity():
    assert _pins.check_alpha_linearity()


@pytest.mark.parametrize("fmt", FMTS)
def test_sampled_equals_full_and_thread_invariance(fmt):
    rng = np.random.default_rng(11)
    M, N, K = 70, 90, 128
    w = _pins.make_w(fmt, M, N, K, rng)
    d, an, bn = oracle.gemm_full(fmt, w, nthreads=3)
    d1, _, _ = oracle.gemm_full(fmt, w, nthreads=1)
    assert np.array_equal(d, d1)
    em = rng.integers(0, M, 500)
    en = rng.integers(0, N, 500)
    ds, ans, bns = oracle.gemm_entries(fmt, w, em, en, nthreads=4)
    assert np.array_equal(ds, d[em, en])
    assert np.array_equal(ans, an[em, en]) and np.array_equal(bns, bn[em, en])


@pytest.mark.parametrize("fmt", FMTS)
def test_row_norms(fmt):
    rng = np.random.default_rng(12)
    w = _pins.make_w(fmt, 6, 7, 64, rng)
    _, an, bn = oracle.gemm_full(fmt, w, nthreads=1)
    va, vb = _pins.ref_values(fmt, w, "A"), _pins.ref_values(fmt, w, "B")
    ta, tb = (w["tA"], w["tB"]) if fmt == "nvfp4" else (1.0, 1.0)
    assert np.allclose(an[:, 0], np.linalg.norm(va, axis=1) * ta, rtol=1e-14, atol=0)
    assert np.allclose(bn[0, :], np.linalg.norm(vb, axis=1) * tb, rtol=1e-14, atol=0)


def test_rejects_bad_arguments():
    w = {"fmt": "mxfp8", "M": 2, "N": 2, "K": 48, "A": np.zeros((2, 48), np.uint8),
         "B": np.zeros((2, 48), np.uint8), "sA": np.zeros((2, 2), np.uint8), "sB": np.zeros((2, 2), np.uint8)}
    with pytest.raises(ValueError):
        oracle.gemm_full("mxfp8", w)
    w2 = {"fmt": "bf16", "M": 2, "N": 2, "K": 8, "A": np.zeros((2, 8), np.uint16), "B": np.zeros((2, 8), np.uint16)}
    with pytest.raises(ValueError):
        oracle.gemm_entries("bf16", w2, [0, 2], [0, 0])


def test_rel_errors_flags_non_finite():
    r = oracle.rel_errors(np.array([1.0, np.nan, np.inf]), np.zeros(3), np.ones(3), np.ones(3))
    assert r[0] == 1.0 and np.isinf(r[1]) and np.isinf(r[2])
