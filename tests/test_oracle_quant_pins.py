"""Pins of the oracle's quantisation recipes against checks that do not reuse
its encoders: torch's float8_e4m3fn conversion (round to nearest even) for
the NVFP4 block scales, a nearest-value search over the decoded code sets
written here for the elements, and the scale exponent rules stated as
inequalities on each block's largest magnitude.  These recipes are the
checkers of the GPU quantisers, so each pin is also shown to catch a planted
mistake in them."""
import numpy as np
import pytest
import torch

import oracle
import synth

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_code(v, grid):
    """Index into an ascending grid of magnitudes of the value nearest |v|,
    ties to the even index (even mantissa), saturating at the last one."""
    a = np.abs(v)
    i = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, len(grid) - 1)
    j = np.minimum(i + 1, len(grid) - 1)
    lo, hi = a - grid[i], grid[j] - a
    pick = np.where(lo < hi, i, np.where(hi < lo, j, np.where(i % 2 == 0, i, j)))
    return np.where(a >= grid[-1], len(grid) - 1, pick)


def _edge_rows(K, rng):
    rows = [rng.standard_normal(K).astype(np.float32) * np.float32(s) for s in (1.0, 1e-2, 1e2)]
    t = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32), K // 8)
    rows.append(t)
    z = rng.standard_normal(K).astype(np.float32)
    z[:16] = 0.0
    z[16:32:2] = -0.0
    rows.append(z)
    return np.stack(rows)


def _nvfp4_independent(x):
    """The NVFP4 recipe recomputed in fp32 with torch: tensor scale
    t = amax / 2688, block scale = float8_e4m3fn(amax_blk / (6 t)),
    elements the nearest E2M1 value of x / (s t)."""
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    rows, K = xt.shape
    amax = xt.abs().max()
    t = amax / torch.tensor(2688.0) if amax > 0 else torch.tensor(1.0)
    blk = xt.reshape(rows, K // 16, 16)
    ab = blk.abs().amax(dim=2)
    v = ab / (torch.tensor(6.0) * t)
    s16 = v.to(torch.float8_e4m3fn)
    sv = s16.to(torch.float32)
    denom = (sv * t).unsqueeze(2)
    q = torch.where(denom > 0, blk / torch.where(denom > 0, denom, torch.ones_like(denom)), blk * 0.0)
    qn = q.reshape(rows, K).numpy().astype(np.float64)
    mag = _nearest_code(qn, E2M1_GRID)
    codes = (mag | np.where(np.signbit(qn), 8, 0)).astype(np.uint8)
    return s16.view(torch.uint8).numpy(), codes, float(t), qn


def _nvfp4_matches(x):
    c, s, t = oracle.quant_nvfp4(x)
    s_ref, codes_ref, t_ref, _ = _nvfp4_independent(x)
    return t == t_ref and np.array_equal(s, s_ref) and np.array_equal(oracle.unpack_fp4(c), codes_ref)


def test_nvfp4_recipe_against_torch_e4m3():
    rng = np.random.default_rng(21)
    for x in (synth.normal(31, 24, 256), np.concatenate([synth.normal(32, 4, 128), _edge_rows(128, rng)])):
        assert _nvfp4_matches(x)


def test_nvfp4_scaled_elements_stay_near_the_grid_top():
    """A block's largest element maps to at most 6 / (1 - 2^-4) before
    rounding (the E4M3 block scale is within 2^-4 of exact), and every code
    is a value of the E2M1 grid, so |q| <= 6."""
    x = synth.normal(33, 40, 512)
    _, _, _, q = _nvfp4_independent(x)
    assert np.abs(q).max() <= 6.0 / (1 - 2.0 ** -4)
    c, _, _ = oracle.quant_nvfp4(x)
    v = oracle.decode("e2m1", oracle.unpack_fp4(c))
    assert np.abs(v).max() <= 6.0 and np.isin(np.abs(v), E2M1_GRID).all()


# scale rule per element: (largest element value, exponent rule, bounds on amax / scale)
MX_RULES = {
    "e4m3": ("ratio", 448.0, (448.0, 896.0)),
    "e5m2": ("ratio", 57344.0, (57344.0, 114688.0)),
    "e2m1": ("ratio", 6.0, (6.0, 12.0)),
    "e2m3": ("ocp", 7.5, (4.0, 8.0)),        # 2^(floor(log2 amax) - 2)
    "e3m2": ("ocp", 28.0, (16.0, 32.0)),     # 2^(floor(log2 amax) - 4)
}


def _mx_scale_rule_holds(elem, x):
    _, s = oracle.quant_mx(x, elem)
    rows, K = x.shape
    amax = np.abs(x.astype(np.float64)).reshape(rows, K // 32, 32).max(axis=2)
    sc = oracle.decode("e8m0", s)
    lo, hi = MX_RULES[elem][2]
    r = amax / sc
    nz = amax > 0
    return bool(np.all((r[nz] >= lo) & (r[nz] < hi)) and np.all(s[~nz] == 127))


@pytest.mark.parametrize("elem", list(MX_RULES))
def test_mx_scale_exponent_rule(elem):
    x = np.concatenate([synth.normal(34, 16, 512), _edge_rows(512, np.random.default_rng(2))])
    assert _mx_scale_rule_holds(elem, x)


def _unpack(elem, c, K):
    if elem == "e2m1":
        return oracle.unpack_fp4(c)
    if elem in ("e2m3", "e3m2"):
        return synth.unpack_fp6_rows(c, K)
    return c


def _only_above_max_saturates(elem, x):
    """Each element is the nearest value of the format's code set to x /
    scale (ties to the even code), so only values beyond the largest one
    saturate."""
    c, s = oracle.quant_mx(x, elem)
    rows, K = x.shape
    codes = _unpack(elem, c, K)
    nbits = {"e2m1": 4, "e2m3": 6, "e3m2": 6}.get(elem, 8)
    sign = 1 << (nbits - 1)
    allv = oracle.decode(elem, np.arange(sign, dtype=np.uint8))       # non-negative codes
    finite = np.isfinite(allv)
    grid, order = allv[finite], np.arange(sign)[finite]
    sc = np.repeat(oracle.decode("e8m0", s), 32, axis=1)
    v = x.astype(np.float64) / sc
    want_mag = order[_nearest_code(v, grid)]
    want = (want_mag | np.where(np.signbit(v), sign, 0)).astype(np.uint8)
    return np.array_equal(codes, want)


@pytest.mark.parametrize("elem", list(MX_RULES))
def test_mx_elements_nearest_and_saturate_only_past_max(elem):
    x = np.concatenate([synth.normal(35, 12, 256), _edge_rows(256, np.random.default_rng(3))])
    assert _only_above_max_saturates(elem, x)


@pytest.mark.parametrize("mut,check", [
    (17, lambda: _mx_scale_rule_holds("e2m3", synth.normal(36, 8, 256))),     # FP6 scale by the ratio rule
    (17, lambda: _mx_scale_rule_holds("e3m2", synth.normal(36, 8, 256))),
    (19, lambda: _mx_scale_rule_holds("e5m2", synth.normal(36, 8, 256))),     # E5M2 with E4M3's emax
    (18, lambda: _nvfp4_matches(synth.normal(37, 8, 256))),                   # block scale truncated
])
def test_planted_recipe_mistakes_are_caught(mut, check):
    assert check()
    oracle.set_mutation(mut)
    try:
        assert not check()
    finally:
        oracle.set_mutation(0)
