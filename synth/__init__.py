"""Seeded synthetic inputs for the block-scaled GEMM workloads.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It draws standard-normal matrices from a fixed PCG64 seed and turns
them into the operand encodings the GEMM consumes:

* BF16: fp32 -> bf16 by round-to-nearest-even on the bit pattern.
* MXFP8 / MXFP4: one power-of-two (E8M0) scale per 32 consecutive K elements,
  ``scale = 2**floor(log2(amax / emax))`` with ``emax`` = 448 (E4M3), 57344
  (E5M2, the OCP format's other 8-bit element) or 6 (E2M1), elements rounded
  to nearest-even on the element grid and saturated.
* NVFP4: one fp32 tensor scale ``t = amax_tensor / (6 * 448)``, one E4M3 scale
  per 16 K elements ``s = RNE_e4m3(amax_block / (6 * t))``, elements
  ``RNE_e2m1(x / (s * t))`` — all divisions and products in fp32.

The element formats are those of the OCP Microscaling (MX) v1.0
specification; the pages name them (ThunderKittens 2.0 notes, "new features"
table: MXFP8/NVFP4; "Dissecting ThunderKittens", tile abstractions: fp8e4m3,
fp8e8m0 and packed fp4e2m1_2 with two FP4 values per byte) but do not define
them.  FP4 packing: element 2j in bits [3:0], element 2j+1 in bits [7:4].

Nothing here decodes a code back to a value or multiplies operands: rounding
is done in the value domain (``_round_*``) and the rounded values are then
bit-packed (``_pack_*``).  The GEMM arithmetic lives only in the HIP kernels
and, independently, in the CPU oracle.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "normal", "bf16_from_f32", "quant_mx", "quant_nvfp4", "workload",
    "sample_entries", "E4M3_MAX", "E2M1_MAX",
]

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
E2M1_MAX = 6.0
E2M3_MAX = 7.5
E3M2_MAX = 28.0


def normal(seed: int, rows: int, cols: int) -> np.ndarray:
    """Standard-normal float32 matrix (rows x cols) from ``PCG64(seed)``."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal((rows, cols), dtype=np.float32)


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


# ---- value-domain rounding onto the element grids (RNE, saturating) --------

def _round_e4m3(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the E4M3 grid (3 mantissa bits, min exponent -6,
    subnormal quantum 2**-9), ties to even, saturate at 448.  Sign kept."""
    a = np.abs(v)
    _, e = np.frexp(a)                   # a in [2**(e-1), 2**e)
    ex = np.maximum(e - 1, -6)           # binade exponent, subnormals share -6
    q = np.ldexp(1.0, ex - 3)            # grid spacing in that binade
    r = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    return np.copysign(r, v)


def _round_e5m2(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the E5M2 grid (2 mantissa bits, min exponent
    -14, subnormal quantum 2**-16), ties to even, saturate at 57344."""
    a = np.abs(v)
    _, e = np.frexp(a)
    ex = np.maximum(e - 1, -14)
    q = np.ldexp(1.0, ex - 2)
    r = np.minimum(np.rint(a / q) * q, E5M2_MAX)
    return np.copysign(r, v)


def _round_e2m1(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6},
    ties to even mantissa, saturate at 6.  Sign kept."""
    a = np.abs(v)
    _, e = np.frexp(a)
    ex = np.maximum(e - 1, 0)            # subnormal binade shares exponent 0
    q = np.ldexp(1.0, ex - 1)            # 1 mantissa bit
    r = np.minimum(np.rint(a / q) * q, E2M1_MAX)
    return np.copysign(r, v)


def _round_grid(v: np.ndarray, mbits: int, emin: int, vmax: float) -> np.ndarray:
    """Round float64 values to a grid with `mbits` mantissa bits and smallest
    normal binade 2**emin (subnormals share its spacing), ties to even,
    saturate at vmax.  Sign kept."""
    a = np.abs(v)
    _, e = np.frexp(a)
    ex = np.maximum(e - 1, emin)
    q = np.ldexp(1.0, ex - mbits)
    r = np.minimum(np.rint(a / q) * q, vmax)
    return np.copysign(r, v)


# ---- bit packing of grid values ---------------------------------------------

def _pack_fp6(r: np.ndarray, mbits: int, bias: int) -> np.ndarray:
    """Grid values -> 6-bit codes (sign in bit 5) of an FP6 format with
    `mbits` mantissa bits and exponent bias `bias`."""
    a = np.abs(r)
    _, e = np.frexp(a)
    ex = e - 1
    normal = a >= 2.0 ** (1 - bias)
    ex_n = np.where(normal, ex, 0)
    man_n = np.where(normal, np.rint((a / np.ldexp(1.0, ex_n) - 1.0) * 2 ** mbits), 0)
    code_n = ((ex_n + bias) << mbits) + man_n.astype(np.int64)
    code_s = np.rint(a / 2.0 ** (1 - bias - mbits)).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = code | np.where(np.signbit(r), 0x20, 0)
    return code.astype(np.uint8)


def pack_fp6_rows(codes: np.ndarray) -> np.ndarray:
    """(rows, K) 6-bit codes -> (rows, 3K/4) bytes: element j of a row at bits
    6j .. 6j+5 of the row's bytes read as one little-endian bit string."""
    c = codes.astype(np.uint32).reshape(codes.shape[0], -1, 4)
    g = c[:, :, 0] | (c[:, :, 1] << 6) | (c[:, :, 2] << 12) | (c[:, :, 3] << 18)
    out = np.stack([g & 0xFF, (g >> 8) & 0xFF, (g >> 16) & 0xFF], axis=2)
    return out.reshape(codes.shape[0], -1).astype(np.uint8)


def unpack_fp6_rows(packed: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_fp6_rows."""
    b = packed.astype(np.uint32).reshape(packed.shape[0], -1, 3)
    g = b[:, :, 0] | (b[:, :, 1] << 8) | (b[:, :, 2] << 16)
    out = np.stack([(g >> (6 * i)) & 0x3F for i in range(4)], axis=2)
    return out.reshape(packed.shape[0], K).astype(np.uint8)




def _pack_e4m3(r: np.ndarray) -> np.ndarray:
    a = np.abs(r)
    _, e = np.frexp(a)
    ex = e - 1
    normal = a >= 2.0 ** -6
    ex_n = np.where(normal, ex, 0)
    man_n = np.where(normal, np.rint((a / np.ldexp(1.0, ex_n) - 1.0) * 8.0), 0)
    code_n = ((ex_n + 7) << 3) + man_n.astype(np.int64)
    code_s = np.rint(a / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = code | np.where(np.signbit(r), 0x80, 0)
    return code.astype(np.uint8)


def _pack_e5m2(r: np.ndarray) -> np.ndarray:
    a = np.abs(r)
    _, e = np.frexp(a)
    ex = e - 1
    normal = a >= 2.0 ** -14
    ex_n = np.where(normal, ex, 0)
    man_n = np.where(normal, np.rint((a / np.ldexp(1.0, ex_n) - 1.0) * 4.0), 0)
    code_n = ((ex_n + 15) << 2) + man_n.astype(np.int64)
    code_s = np.rint(a / 2.0 ** -16).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = code | np.where(np.signbit(r), 0x80, 0)
    return code.astype(np.uint8)


def _pack_e2m1(r: np.ndarray) -> np.ndarray:
    a = np.abs(r)
    _, e = np.frexp(a)
    ex = e - 1
    normal = a >= 1.0
    ex_n = np.where(normal, ex, 0)
    man_n = np.where(normal, np.rint((a / np.ldexp(1.0, ex_n) - 1.0) * 2.0), 0)
    code_n = ((ex_n + 1) << 1) + man_n.astype(np.int64)
    code_s = np.rint(a * 2.0).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = code | np.where(np.signbit(r), 0x8, 0)
    return code.astype(np.uint8)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """(rows, K) 4-bit codes -> (rows, K/2) bytes, even k in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def _floor_log2_ratio(amax: np.ndarray, emax: float) -> np.ndarray:
    """Exact floor(log2(amax / emax)) for amax > 0, via frexp of both."""
    fa, ea = np.frexp(amax.astype(np.float64))
    fe, ee = np.frexp(emax)
    return (ea - ee) - (fa < fe).astype(np.int64)


def quant_mx(x: np.ndarray, elem: str) -> tuple[np.ndarray, np.ndarray]:
    """MX quantisation along the last axis (K), 32-element blocks.

    Returns ``(codes, scales)``: for ``elem='e4m3'`` or ``'e5m2'`` codes are
    (rows, K) uint8; for ``elem='e2m1'`` they are (rows, K/2) uint8 with two
    elements per byte; for the FP6 ``'e2m3'`` / ``'e3m2'`` (rows, 3K/4) uint8,
    four elements per three bytes (pack_fp6_rows).
    ``scales`` are (rows, K/32) E8M0 codes.  An all-zero block gets scale code
    127 (1.0) and zero elements.
    """
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32 for MX formats")
    # scale reference: the element's largest value, except for FP6, whose
    # scales follow the OCP recipe 2^(floor(log2 amax) - emax) (emax 2 / 4)
    emax = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX, "e2m1": E2M1_MAX, "e2m3": 4.0, "e3m2": 16.0}[elem]
    xb = x.astype(np.float64).reshape(rows, K // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    e = np.where(amax > 0, _floor_log2_ratio(np.where(amax > 0, amax, 1.0), emax), 0)
    e = np.clip(e, -127, 127)
    v = xb / np.ldexp(1.0, e)[:, :, None]        # exact: power-of-two divisor
    if elem == "e4m3":
        codes = _pack_e4m3(_round_e4m3(v)).reshape(rows, K)
    elif elem == "e5m2":
        codes = _pack_e5m2(_round_e5m2(v)).reshape(rows, K)
    elif elem == "e2m1":
        codes = _pack_nibbles(_pack_e2m1(_round_e2m1(v)).reshape(rows, K))
    elif elem == "e2m3":
        codes = pack_fp6_rows(_pack_fp6(_round_grid(v, 3, 0, E2M3_MAX), 3, 1).reshape(rows, K))
    elif elem == "e3m2":
        codes = pack_fp6_rows(_pack_fp6(_round_grid(v, 2, -2, E3M2_MAX), 2, 3).reshape(rows, K))
    else:
        raise ValueError(elem)
    return codes, (e + 127).astype(np.uint8)


def quant_nvfp4(x: np.ndarray) -> tuple[np.ndarray, np.ndarray, float]:
    """NVFP4 quantisation: E2M1 elements, E4M3 scale per 16 along K, one fp32
    tensor scale.  Returns ``(codes (rows, K/2) uint8, scales (rows, K/16)
    uint8, t float)``.  Every step is carried out in fp32."""
    rows, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16 for NVFP4")
    x = np.ascontiguousarray(x, dtype=np.float32)
    f32 = np.float32
    amax_t = f32(np.max(np.abs(x))) if x.size else f32(0)
    t = amax_t / f32(E2M1_MAX * E4M3_MAX) if amax_t > 0 else f32(1.0)
    xb = x.reshape(rows, K // 16, 16)
    amax_b = np.max(np.abs(xb), axis=2)
    v = amax_b / (f32(E2M1_MAX) * t)                      # fp32
    s_val = _round_e4m3(v.astype(np.float64))              # grid value
    s_codes = _pack_e4m3(s_val)
    denom = (s_val.astype(np.float32) * t)[:, :, None]     # fp32
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(denom > 0, xb / np.where(denom > 0, denom, f32(1)), xb * f32(0))
    q = q.astype(np.float32)
    e_codes = _pack_e2m1(_round_e2m1(q.astype(np.float64))).reshape(rows, K)
    return _pack_nibbles(e_codes), s_codes.astype(np.uint8), float(t)


# ---- the benchmark workloads --------------------------------------------------

def workload(fmt: str, M: int, N: int, K: int, seed_a: int, seed_b: int,
             elem_a: str = "e4m3", elem_b: str = "e4m3") -> dict:
    """Encoded operands for one GEMM D = A . B^T of the given format.

    Returns a dict with numpy arrays ``A``, ``B`` (and ``sA``, ``sB``, ``tA``,
    ``tB`` where the format has scales).  A is M x K, B is N x K, K-major.
    For ``fmt='mxfp8'`` each operand's MX element format is ``elem_a`` /
    ``elem_b`` ('e4m3', 'e5m2', 'e2m1', 'e2m3' or 'e3m2'), recorded as
    ``elemA`` / ``elemB``.
    """
    xa = normal(seed_a, M, K)
    xb = normal(seed_b, N, K)
    out = {"fmt": fmt, "M": M, "N": N, "K": K}
    if fmt == "bf16":
        out["A"], out["B"] = bf16_from_f32(xa), bf16_from_f32(xb)
    elif fmt in ("mxfp8", "mxfp4"):
        ea, eb = (elem_a, elem_b) if fmt == "mxfp8" else ("e2m1", "e2m1")
        out["A"], out["sA"] = quant_mx(xa, ea)
        out["B"], out["sB"] = quant_mx(xb, eb)
        if fmt == "mxfp8":
            out["elemA"], out["elemB"] = ea, eb
    elif fmt == "nvfp4":
        out["A"], out["sA"], out["tA"] = quant_nvfp4(xa)
        out["B"], out["sB"], out["tB"] = quant_nvfp4(xb)
    else:
        raise ValueError(fmt)
    return out


def sample_entries(seed: int, M: int, N: int, count: int = 4096) -> tuple[np.ndarray, np.ndarray]:
    """Output entries checked at large shapes: the structured rows/cols
    {0, 255, 256, last} crossed (deduplicated, in range), then uniform draws
    from ``PCG64(seed)`` up to ``count`` entries in total."""
    rs = sorted({r for r in (0, 255, 256, M - 1) if 0 <= r < M})
    cs = sorted({c for c in (0, 255, 256, N - 1) if 0 <= c < N})
    em = [r for r in rs for _ in cs]
    en = [c for _ in rs for c in cs]
    g = np.random.Generator(np.random.PCG64(seed))
    rest = max(0, count - len(em))
    em = np.concatenate([np.array(em, dtype=np.int64), g.integers(0, M, rest, dtype=np.int64)])
    en = np.concatenate([np.array(en, dtype=np.int64), g.integers(0, N, rest, dtype=np.int64)])
    return em, en
