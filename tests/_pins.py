"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check returns True/False so that the same battery can be run with a
planted mistake switched on in the oracle (the mutation tests expect at least
one check to fail for every planted mistake).

Independent value sources:
  * E4M3 and E8M0 code values: torch's float8_e4m3fn / float8_e8m0fnu dtypes
    (a third-party decoder) and the OCP MX v1.0 anchor tables in tests/golden.
  * E2M1 code values: the OCP MX v1.0 E2M1 table in tests/golden.
  * bf16 values: the IEEE binary32 reinterpretation of (bits << 16) by numpy.
  * Sums: exact rationals (fractions.Fraction) or numpy float64 matmuls of
    inputs whose every partial sum is exact in fp64.
"""
from __future__ import annotations

from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

import oracle
import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


def _table(name):
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        out[int(c, 16)] = float(v)
    return out


E2M1_TABLE = _table("ocp_e2m1.txt")


def ref_e2m1(codes):
    c = np.asarray(codes, np.uint8)
    mag = np.array([E2M1_TABLE[i] for i in range(8)])[c & 7]
    return np.where(c & 8, -mag, mag)


def ref_e4m3(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def ref_e5m2(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e5m2).to(torch.float64).numpy()


def ref_e8m0(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def ref_bf16(bits):
    b = np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def ref_values(fmt, w, which):
    """Independently decoded, block-scaled values of operand 'A' or 'B' (rows x K)."""
    X = w[which]
    K = w["K"]
    if fmt == "bf16":
        return ref_bf16(X)
    if fmt == "mxfp8" and w.get("elem" + which, "e4m3") != "e2m1":
        el = ref_e5m2(X) if w.get("elem" + which, "e4m3") == "e5m2" else ref_e4m3(X)
        sc = ref_e8m0(w["s" + which])
        return el * np.repeat(sc, 32, axis=1)
    codes = np.empty((X.shape[0], K), np.uint8)
    codes[:, 0::2] = X & 0xF
    codes[:, 1::2] = X >> 4
    el = ref_e2m1(codes)
    if fmt in ("mxfp4", "mxfp8"):          # E2M1 elements of an MX operand
        return el * np.repeat(ref_e8m0(w["s" + which]), 32, axis=1)
    return el * np.repeat(ref_e4m3(w["s" + which]), 16, axis=1)


# ---- random encoded operands spanning the code ranges -------------------------

def random_codes(fmt, rows, K, rng, scale_lo=0, scale_hi=254, finite=True, bf16_exp=(100, 154)):
    """Random operand codes over (nearly) the whole code range."""
    if fmt == "bf16":
        sign = rng.integers(0, 2, (rows, K)) << 15
        exp = rng.integers(bf16_exp[0], bf16_exp[1], (rows, K)) << 7    # finite, normal
        man = rng.integers(0, 128, (rows, K))
        return {"X": (sign | exp | man).astype(np.uint16)}
    if fmt == "mxfp8":
        c = rng.integers(0, 256, (rows, K)).astype(np.uint8)
        if finite:
            c[(c & 0x7F) == 0x7F] = 0x3F
        s = rng.integers(scale_lo, scale_hi + 1, (rows, K // 32)).astype(np.uint8)
        return {"X": c, "s": s}
    c = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    if fmt == "mxfp4":
        s = rng.integers(scale_lo, scale_hi + 1, (rows, K // 32)).astype(np.uint8)
    else:
        s = rng.integers(scale_lo, min(scale_hi, 0x7E) + 1, (rows, K // 16)).astype(np.uint8)
    return {"X": c, "s": s}


def random_e5m2(rows, K, rng, exp=(0, 31)):
    """Random finite E5M2 codes with exponent fields in [exp[0], exp[1])
    (the all-ones field, infinities and NaNs, is never drawn)."""
    sign = rng.integers(0, 2, (rows, K)) << 7
    e = rng.integers(exp[0], min(exp[1], 31), (rows, K)) << 2
    return (sign | e | rng.integers(0, 4, (rows, K))).astype(np.uint8)


def make_w_mx8(elem_a, elem_b, M, N, K, rng, scale_lo=0, scale_hi=254, narrow=False):
    """An MX 8-bit workload whose operands carry elements elem_a / elem_b
    ('e4m3' or 'e5m2') with random E8M0 scales; `narrow` keeps E5M2 codes
    within 2^-5 .. 2^6 so that products span few enough binades for exact
    fp64 sums."""
    w = {"fmt": "mxfp8", "M": M, "N": N, "K": K, "elemA": elem_a, "elemB": elem_b}
    for X, rows, el in (("A", M, elem_a), ("B", N, elem_b)):
        if el == "e5m2":
            w[X] = random_e5m2(rows, K, rng, (10, 21) if narrow else (0, 31))
        elif el == "e2m1":
            w[X] = random_codes("mxfp4", rows, K, rng)["X"]
        elif el in ("e2m3", "e3m2"):
            w[X] = synth.pack_fp6_rows(rng.integers(0, 64, (rows, K), dtype=np.uint8))
        else:
            w[X] = random_codes("mxfp8", rows, K, rng)["X"]
        w["s" + X] = rng.integers(scale_lo, scale_hi + 1, (rows, K // 32)).astype(np.uint8)
    return w


def check_mixed_fraction(elem_a, elem_b, seed=20, M=3, N=4, K=96, exact_scales=False):
    """Per-operand MX element formats against exact rational dot products of
    independently decoded values (torch's float8 types).  With narrow scales
    and E5M2 codes every product has at most 8 significant bits and lies in
    2^-30 .. 2^21, so every fp64 partial sum is exact and equality is
    required; otherwise the fp64 recursive-summation bound is used."""
    rng = np.random.default_rng(seed)
    kw = {"scale_lo": 124, "scale_hi": 130, "narrow": True} if exact_scales else {}
    w = make_w_mx8(elem_a, elem_b, M, N, K, rng, **kw)
    va, vb = ref_values("mxfp8", w, "A"), ref_values("mxfp8", w, "B")
    d, _, _ = oracle.gemm_full("mxfp8", w, nthreads=2)
    if not np.all(np.isfinite(d)):
        return False
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(va[m, k])) * Fraction(float(vb[n, k])) for k in range(K)]
            exact = sum(terms)
            got = Fraction(float(d[m, n]))
            if exact_scales:
                if got != exact:
                    return False
            elif abs(got - exact) > sum(abs(t) for t in terms) * Fraction(K + 2, 2 ** 52):
                return False
    return True


def make_w(fmt, M, N, K, rng, **kw):
    a = random_codes(fmt, M, K, rng, **kw)
    b = random_codes(fmt, N, K, rng, **kw)
    w = {"fmt": fmt, "M": M, "N": N, "K": K, "A": a["X"], "B": b["X"]}
    if fmt != "bf16":
        w["sA"], w["sB"] = a["s"], b["s"]
    if fmt == "nvfp4":
        w["tA"], w["tB"] = float(np.float32(rng.uniform(0.25, 3.0))), float(np.float32(rng.uniform(0.25, 3.0)))
    return w


# ---- checks -------------------------------------------------------------------

def check_brute_force_fraction(fmt, seed=0, M=3, N=4, K=64, exact_scales=False):
    """Oracle vs exact rational dot products (values from independent decoders).
    With a narrow scale range every fp64 partial sum is exact, so equality is
    required; otherwise the fp64 recursive-summation bound is used."""
    rng = np.random.default_rng(seed)
    kw = {"scale_lo": 120, "scale_hi": 134} if exact_scales else {}
    if fmt == "nvfp4" and exact_scales:
        kw = {"scale_lo": 0x30, "scale_hi": 0x48}
    if fmt == "bf16" and exact_scales:
        kw = {"bf16_exp": (124, 132)}       # every partial sum exact in fp64
    w = make_w(fmt, M, N, K, rng, **kw)
    va, vb = ref_values(fmt, w, "A"), ref_values(fmt, w, "B")
    alpha = Fraction(w.get("tA", 1.0)) * Fraction(w.get("tB", 1.0)) if fmt == "nvfp4" else Fraction(1)
    d, _, _ = oracle.gemm_full(fmt, w, nthreads=2)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(va[m, k])) * Fraction(float(vb[n, k])) for k in range(K)]
            exact = alpha * sum(terms)
            if exact_scales and fmt != "nvfp4":
                if Fraction(float(d[m, n])) != exact:
                    return False
            else:
                bound = abs(alpha) * sum(abs(t) for t in terms) * Fraction(K + 2, 2 ** 52)
                if abs(Fraction(float(d[m, n])) - exact) > bound:
                    return False
    return True


def check_identity(fmt, seed=1, M=8, K=64):
    """B = identity (N = K): D[m, n] = value of A[m, n] times B's unit scale."""
    rng = np.random.default_rng(seed)
    a = random_codes(fmt, M, K, rng, scale_lo=110, scale_hi=140)
    N = K
    w = {"fmt": fmt, "M": M, "N": N, "K": K, "A": a["X"]}
    if fmt == "bf16":
        B = np.zeros((N, K), np.uint16)
        B[np.arange(N), np.arange(K)] = 0x3F80          # 1.0
    elif fmt == "mxfp8":
        B = np.zeros((N, K), np.uint8)
        B[np.arange(N), np.arange(K)] = 0x38            # 1.0
    else:
        codes = np.zeros((N, K), np.uint8)
        codes[np.arange(N), np.arange(K)] = 0x2         # 1.0
        B = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w["B"] = B
    if fmt in ("mxfp8", "mxfp4"):
        w["sA"], w["sB"] = a["s"], np.full((N, K // 32), 127, np.uint8)
    elif fmt == "nvfp4":
        w["sA"], w["sB"] = a["s"], np.full((N, K // 16), 0x38, np.uint8)
        w["tA"], w["tB"] = 1.0, 1.0
    d, _, _ = oracle.gemm_full(fmt, w, nthreads=1)
    return bool(np.array_equal(d, ref_values(fmt, w, "A")))


def check_permutation(fmt, seed=2, M=8, K=128):
    """B[n, k] = 1 iff k = pi(n) with pi crossing scale blocks:
    D[m, n] = dA[m, pi(n)] * sB[n, pi(n)/bs]."""
    rng = np.random.default_rng(seed)
    N = K
    pi = rng.permutation(K)
    a = random_codes(fmt, M, K, rng, scale_lo=110, scale_hi=140)
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
        w["sB"] = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    elif fmt == "nvfp4":
        w["sA"] = a["s"]
        w["sB"] = rng.integers(0x30, 0x48, (N, K // 16)).astype(np.uint8)
        w["tA"], w["tB"] = 1.0, 1.0
    d, _, _ = oracle.gemm_full(fmt, w, nthreads=1)
    va = ref_values(fmt, w, "A")
    vb = ref_values(fmt, w, "B")
    expect = va[:, pi] * vb[np.arange(N), pi][None, :]
    return bool(np.array_equal(d, expect))


def check_pow2_scale_shift(fmt, seed=3, M=5, N=6, K=96, j=3):
    """Adding j to every A scale code (E8M0) multiplies D by exactly 2**j; for
    NVFP4 adding 8*j to the E4M3 exponent field does the same."""
    if fmt == "bf16":
        return True
    rng = np.random.default_rng(seed)
    w = make_w(fmt, M, N, K, rng, scale_lo=100, scale_hi=140)
    if fmt == "nvfp4":
        w["sA"] = rng.integers(0x20, 0x40, (M, K // 16)).astype(np.uint8)
    d0, _, _ = oracle.gemm_full(fmt, w, nthreads=1)
    w2 = dict(w)
    w2["sA"] = (w["sA"].astype(np.int64) + (8 * j if fmt == "nvfp4" else j)).astype(np.uint8)
    d1, _, _ = oracle.gemm_full(fmt, w2, nthreads=1)
    return bool(np.array_equal(d1, d0 * 2.0 ** j))


def check_unit_scale_matmul(fmt, seed=4, M=16, N=24, K=256):
    """With unit scales the GEMM is a plain matmul of decoded elements.  The
    element grids make every partial sum exact in fp64 here, so numpy's
    float64 matmul (any summation order) must agree bit for bit."""
    rng = np.random.default_rng(seed)
    if fmt == "bf16":
        return True
    w = make_w(fmt, M, N, K, rng)
    if fmt in ("mxfp8", "mxfp4"):
        w["sA"] = np.full_like(w["sA"], 127)
        w["sB"] = np.full_like(w["sB"], 127)
    else:
        w["sA"] = np.full_like(w["sA"], 0x38)
        w["sB"] = np.full_like(w["sB"], 0x38)
        w["tA"], w["tB"] = 1.0, 1.0
    d, _, _ = oracle.gemm_full(fmt, w, nthreads=2)
    if fmt == "mxfp8":
        ea, eb = ref_e4m3(w["A"]), ref_e4m3(w["B"])
    else:
        ca = np.empty((M, K), np.uint8); ca[:, 0::2] = w["A"] & 0xF; ca[:, 1::2] = w["A"] >> 4
        cb = np.empty((N, K), np.uint8); cb[:, 0::2] = w["B"] & 0xF; cb[:, 1::2] = w["B"] >> 4
        ea, eb = ref_e2m1(ca), ref_e2m1(cb)
    return bool(np.array_equal(d, ea @ eb.T))


def check_bf16_integers(seed=5, M=24, N=20, K=512):
    """bf16 operands holding integers in [-8, 8]: D equals the int64 matmul."""
    rng = np.random.default_rng(seed)
    ia = rng.integers(-8, 9, (M, K))
    ib = rng.integers(-8, 9, (N, K))
    fa = ia.astype(np.float32).view(np.uint32) >> 16
    fb = ib.astype(np.float32).view(np.uint32) >> 16
    w = {"fmt": "bf16", "M": M, "N": N, "K": K, "A": fa.astype(np.uint16), "B": fb.astype(np.uint16)}
    d, _, _ = oracle.gemm_full("bf16", w, nthreads=2)
    return bool(np.array_equal(d, (ia @ ib.T).astype(np.float64)))


def check_rectangular_bf16(seed=6, M=5, N=7, K=11):
    """Non-square bf16 case against exact rationals (catches A*B vs A*B^T)."""
    rng = np.random.default_rng(seed)
    ia = rng.integers(-4, 5, (M, K)).astype(np.float32)
    ib = rng.integers(-4, 5, (N, K)).astype(np.float32)
    w = {"fmt": "bf16", "M": M, "N": N, "K": K,
         "A": (ia.view(np.uint32) >> 16).astype(np.uint16),
         "B": (ib.view(np.uint32) >> 16).astype(np.uint16)}
    d, _, _ = oracle.gemm_full("bf16", w, nthreads=1)
    return bool(np.array_equal(d, ia.astype(np.float64) @ ib.astype(np.float64).T))


def check_transpose_symmetry(fmt, seed=7, M=9, N=13, K=64):
    """gemm(A, B) == gemm(B, A)^T bit for bit."""
    rng = np.random.default_rng(seed)
    w = make_w(fmt, M, N, K, rng)
    wt = dict(w)
    wt["M"], wt["N"], wt["A"], wt["B"] = N, M, w["B"], w["A"]
    if fmt != "bf16":
        wt["sA"], wt["sB"] = w["sB"], w["sA"]
    if fmt == "nvfp4":
        wt["tA"], wt["tB"] = w["tB"], w["tA"]
    d1, _, _ = oracle.gemm_full(fmt, w, nthreads=1)
    d2, _, _ = oracle.gemm_full(fmt, wt, nthreads=1)
    return bool(np.array_equal(d1, d2.T))


def check_alpha_linearity(seed=8, M=4, N=5, K=64):
    """NVFP4: D(tA=2, tB=3) == 6 * D(tA=1, tB=1) exactly."""
    rng = np.random.default_rng(seed)
    w = make_w("nvfp4", M, N, K, rng, scale_lo=0x30, scale_hi=0x48)
    w["tA"], w["tB"] = 1.0, 1.0
    d1, _, _ = oracle.gemm_full("nvfp4", w, nthreads=1)
    w["tA"], w["tB"] = 2.0, 3.0
    d6, _, _ = oracle.gemm_full("nvfp4", w, nthreads=1)
    return bool(np.array_equal(d6, 6.0 * d1))


def check_decoders():
    """Oracle decoders vs torch (E4M3/E8M0, all 256 codes), the OCP E2M1
    table (16 codes) and numpy's binary32 view (bf16 samples)."""
    codes = np.arange(256, dtype=np.uint8)
    ok = True
    for fmt, ref in (("e4m3", ref_e4m3), ("e5m2", ref_e5m2), ("e8m0", ref_e8m0)):
        got = oracle.decode(fmt, codes)
        exp = ref(codes)
        ok &= bool(np.array_equal(np.isnan(got), np.isnan(exp)))
        fin = ~np.isnan(exp)
        ok &= bool(np.array_equal(got[fin], exp[fin]))
        ok &= bool(np.array_equal(np.signbit(got[fin]), np.signbit(exp[fin])))
    c16 = np.arange(16, dtype=np.uint8)
    got = oracle.decode("e2m1", c16)
    ok &= bool(np.array_equal(got, ref_e2m1(c16))) and bool(np.array_equal(np.signbit(got), c16 >= 8))
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("bf16", bits)
    exp = ref_bf16(bits)
    fin = ~np.isnan(exp)
    ok &= bool(np.array_equal(got[fin], exp[fin])) and bool(np.array_equal(np.isnan(got), ~fin))
    return ok


def battery():
    """All GEMM/decoder pins; returns {name: passed}."""
    res = {"decoders": check_decoders(),
           "bf16_integers": check_bf16_integers(),
           "bf16_rectangular": check_rectangular_bf16(),
           "nvfp4_alpha": check_alpha_linearity()}
    for fmt in ("bf16", "mxfp8", "mxfp4", "nvfp4"):
        res[f"{fmt}_fraction"] = check_brute_force_fraction(fmt)
        res[f"{fmt}_fraction_exact"] = check_brute_force_fraction(fmt, seed=10, exact_scales=True)
        res[f"{fmt}_identity"] = check_identity(fmt)
        res[f"{fmt}_permutation"] = check_permutation(fmt)
        res[f"{fmt}_pow2"] = check_pow2_scale_shift(fmt)
        res[f"{fmt}_unit_matmul"] = check_unit_scale_matmul(fmt)
        res[f"{fmt}_transpose"] = check_transpose_symmetry(fmt)
    for ea, eb in (("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e4m3", "e2m1"), ("e2m1", "e5m2")):
        res[f"mx8_{ea}x{eb}_fraction"] = check_mixed_fraction(ea, eb)
        res[f"mx8_{ea}x{eb}_fraction_exact"] = check_mixed_fraction(ea, eb, seed=21, exact_scales=True)
    return res
