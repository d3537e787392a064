"""Plain fp64 CPU oracle for the block-scaled GEMM D = alpha * (sA.A) (sB.B)^T.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product path (the HIP library
and its Python binding) never imports, loads or calls anything here, and this
package never imports the product.

The arithmetic lives in ``oracle.c`` (built into ``liboracle.so`` by
``oracle/build.py``); this module only marshals numpy arrays.  Kinds:
0 = BF16, 1 = MXFP8, 2 = MXFP4, 3 = NVFP4, 4 / 5 / 6 = MX with E5M2 / E2M3 /
E3M2 elements.  For fmt 'mxfp8' a workload may name each operand's MX element
format in w['elemA'] / w['elemB'] ('e4m3', the default, 'e5m2', 'e2m1' packed
two per byte, or 'e2m3' / 'e3m2' packed four per three bytes).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "liboracle.so"

KINDS = {"bf16": 0, "mxfp8": 1, "mxfp4": 2, "nvfp4": 3}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(str(LIB_PATH))
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_decode_e2m1.restype = ctypes.c_double
    lib.orc_decode_e4m3.restype = ctypes.c_double
    lib.orc_decode_e8m0.restype = ctypes.c_double
    lib.orc_decode_bf16.restype = ctypes.c_double
    lib.orc_decode_e5m2.restype = ctypes.c_double
    lib.orc_decode_e2m3.restype = ctypes.c_double
    lib.orc_decode_e3m2.restype = ctypes.c_double
    for f in (lib.orc_decode_e2m1, lib.orc_decode_e4m3, lib.orc_decode_e8m0, lib.orc_decode_bf16,
              lib.orc_decode_e5m2, lib.orc_decode_e2m3, lib.orc_decode_e3m2):
        f.argtypes = [ctypes.c_uint]
    lib.orc_fp6_get.argtypes = [P, I64]
    lib.orc_fp6_get.restype = ctypes.c_uint
    for f in (lib.orc_encode_e2m1, lib.orc_encode_e4m3, lib.orc_encode_bf16, lib.orc_encode_e5m2,
              lib.orc_encode_e2m3, lib.orc_encode_e3m2):
        f.argtypes = [ctypes.c_double]
        f.restype = ctypes.c_uint
    lib.orc_decode_array.argtypes = [ctypes.c_int, P, I64, P]
    lib.orc_encode_array.argtypes = [ctypes.c_int, P, I64, P]
    lib.orc_set_mutation.argtypes = [ctypes.c_int]
    lib.orc_gemm_entries2.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_double, P, P, ctypes.c_double,
                                      I64, I64, I64, P, P, I64, P, P, P, ctypes.c_int]
    lib.orc_gemm_entries2.restype = ctypes.c_int
    lib.orc_gemm_full2.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_double, P, P, ctypes.c_double,
                                   I64, I64, I64, P, P, P, ctypes.c_int]
    lib.orc_gemm_full2.restype = ctypes.c_int
    lib.orc_quant_mx.argtypes = [ctypes.c_int, P, I64, I64, P, P]
    lib.orc_quant_mx.restype = ctypes.c_int
    lib.orc_quant_nvfp4.argtypes = [P, I64, I64, P, P, P]
    lib.orc_quant_nvfp4.restype = ctypes.c_int
    lib.orc_quant_bf16.argtypes = [P, I64, P]
    lib.orc_requant_nvfp4_mx8.argtypes = [P, P, I64, I64, P, P]
    lib.orc_requant_nvfp4_mx8.restype = ctypes.c_int
    lib.orc_requant_nvfp4_e2m3.argtypes = [P, P, I64, I64, P, P]
    lib.orc_requant_nvfp4_e2m3.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def set_mutation(m: int) -> None:
    """Planted-mistake switch used by the pin tests (0 = off)."""
    _load().orc_set_mutation(int(m))


# ---- formats -------------------------------------------------------------

def decode(fmt: str, codes) -> np.ndarray:
    """Decode codes to float64: fmt in {'e2m1', 'e4m3', 'e5m2', 'e2m3', 'e3m2', 'e8m0', 'bf16'}
    (one code per array element)."""
    lib = _load()
    idx = {"e2m1": 0, "e4m3": 1, "e8m0": 2, "bf16": 3, "e5m2": 4, "e2m3": 5, "e3m2": 6}[fmt]
    c = _c(codes, np.uint16 if fmt == "bf16" else np.uint8).ravel()
    out = np.empty(c.size, dtype=np.float64)
    lib.orc_decode_array(idx, _ptr(c), c.size, _ptr(out))
    return out.reshape(np.shape(codes))


def encode(fmt: str, x) -> np.ndarray:
    """Nearest-even encode of float64 values: fmt in {'e2m1','e4m3','e5m2','e2m3','e3m2','bf16'}."""
    lib = _load()
    idx = {"e2m1": 0, "e4m3": 1, "bf16": 3, "e5m2": 4, "e2m3": 5, "e3m2": 6}[fmt]
    v = _c(x, np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint16 if fmt == "bf16" else np.uint8)
    lib.orc_encode_array(idx, _ptr(v), v.size, _ptr(out))
    return out.reshape(np.shape(x))


def unpack_fp6(packed: np.ndarray, K: int) -> np.ndarray:
    """(rows, 3K/4) bytes -> (rows, K) FP6 codes, as the oracle reads them."""
    lib = _load()
    p = _c(packed, np.uint8)
    rows = p.shape[0]
    out = np.empty((rows, K), np.uint8)
    for r in range(rows):
        row = np.ascontiguousarray(p[r])
        for j in range(K):
            out[r, j] = lib.orc_fp6_get(_ptr(row), j)
    return out


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """(rows, K/2) bytes -> (rows, K) E2M1 codes, element 2j = low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---- GEMM ----------------------------------------------------------------

_MX8 = {"e4m3": 1, "e5m2": 4, "e2m1": 2, "e2m3": 5, "e3m2": 6}


def _operands(fmt, w):
    """(kind of A, kind of B, A, sA, tA, B, sB, tB) of workload w."""
    kind = KINDS[fmt]
    if fmt == "bf16":
        A, B = _c(w["A"], np.uint16), _c(w["B"], np.uint16)
        return kind, kind, A, None, 1.0, B, None, 1.0
    ka = kb = kind
    if fmt == "mxfp8":
        ka, kb = _MX8[w.get("elemA", "e4m3")], _MX8[w.get("elemB", "e4m3")]
    A, B = _c(w["A"], np.uint8), _c(w["B"], np.uint8)
    sA, sB = _c(w["sA"], np.uint8), _c(w["sB"], np.uint8)
    return ka, kb, A, sA, float(w.get("tA", 1.0)), B, sB, float(w.get("tB", 1.0))


def gemm_entries(fmt: str, w: dict, em, en, nthreads: int | None = None):
    """D_ref and the per-entry row norms at entries (em[i], en[i]).

    ``w`` holds the encoded operands (keys A, B, sA, sB, tA, tB, M, N, K as
    produced by ``synth.workload``).  Returns ``(d, anorm, bnorm)`` float64
    arrays, with ``anorm = ||dA_m|| * |tA|`` and ``bnorm = ||dB_n|| * |tB|``.
    """
    lib = _load()
    ka, kb, A, sA, tA, B, sB, tB = _operands(fmt, w)
    em = _c(em, np.int64)
    en = _c(en, np.int64)
    n = em.size
    d = np.empty(n, np.float64)
    an = np.empty(n, np.float64)
    bn = np.empty(n, np.float64)
    rc = lib.orc_gemm_entries2(ka, kb, _ptr(A), _ptr(sA), tA, _ptr(B), _ptr(sB), tB,
                              w["M"], w["N"], w["K"], _ptr(em), _ptr(en), n,
                              _ptr(d), _ptr(an), _ptr(bn), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return d, an, bn


def gemm_full(fmt: str, w: dict, nthreads: int | None = None, norms: bool = True):
    """All M x N entries of D_ref (row-major) and, if ``norms``, the norms."""
    lib = _load()
    ka, kb, A, sA, tA, B, sB, tB = _operands(fmt, w)
    M, N = w["M"], w["N"]
    d = np.empty((M, N), np.float64)
    an = np.empty((M, N), np.float64) if norms else None
    bn = np.empty((M, N), np.float64) if norms else None
    rc = lib.orc_gemm_full2(ka, kb, _ptr(A), _ptr(sA), tA, _ptr(B), _ptr(sB), tB,
                           M, N, w["K"], _ptr(d), _ptr(an), _ptr(bn),
                           nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return d, an, bn


# ---- quantisation recipes (to confirm the input generator) -----------------

def quant_mx(x: np.ndarray, elem: str):
    lib = _load()
    x = _c(x, np.float32)
    rows, K = x.shape
    width = {"e2m1": K // 2, "e2m3": K // 4 * 3, "e3m2": K // 4 * 3}.get(elem, K)
    codes = np.zeros((rows, width), np.uint8)
    scales = np.zeros((rows, K // 32), np.uint8)
    idx = {"e2m1": 0, "e4m3": 1, "e5m2": 2, "e2m3": 3, "e3m2": 4}[elem]
    if lib.orc_quant_mx(idx, _ptr(x), rows, K, _ptr(codes), _ptr(scales)):
        raise ValueError("bad K")
    return codes, scales


def quant_nvfp4(x: np.ndarray):
    lib = _load()
    x = _c(x, np.float32)
    rows, K = x.shape
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, K // 16), np.uint8)
    t = np.zeros(1, np.float32)
    if lib.orc_quant_nvfp4(_ptr(x), rows, K, _ptr(codes), _ptr(scales), _ptr(t)):
        raise ValueError("bad K")
    return codes, scales, float(t[0])


def quant_bf16(x: np.ndarray) -> np.ndarray:
    lib = _load()
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.orc_quant_bf16(_ptr(x), x.size, _ptr(out))
    return out


def requant_nvfp4_mx8(codes: np.ndarray, scales: np.ndarray, K: int):
    """NVFP4 operand (rows x K/2 packed E2M1, rows x K/16 E4M3) -> the MXFP8
    operand of the FP8-rate GEMM (rows x K E4M3, rows x K/32 E8M0)."""
    lib = _load()
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint8)
    rows = c.shape[0]
    out = np.zeros((rows, K), np.uint8)
    osc = np.zeros((rows, K // 32), np.uint8)
    if lib.orc_requant_nvfp4_mx8(_ptr(c), _ptr(s), rows, K, _ptr(out), _ptr(osc)):
        raise ValueError("K must be a multiple of 32")
    return out, osc


def requant_nvfp4_e2m3(codes: np.ndarray, scales: np.ndarray, K: int):
    """NVFP4 operand (rows x K/2 packed E2M1, rows x K/16 E4M3) -> the MXFP6
    operand of the FP4-rate GEMM (rows x 3K/4 packed E2M3, rows x K/32 E8M0)."""
    lib = _load()
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint8)
    rows = c.shape[0]
    out = np.zeros((rows, K // 4 * 3), np.uint8)
    osc = np.zeros((rows, K // 32), np.uint8)
    if lib.orc_requant_nvfp4_e2m3(_ptr(c), _ptr(s), rows, K, _ptr(out), _ptr(osc)):
        raise ValueError("K must be a multiple of 32")
    return out, osc


def nvfp4_fp6_workload(w: dict) -> dict:
    """The MXFP6 (E2M3) workload the FP4-rate NVFP4 GEMM computes for NVFP4
    workload w (its D is this workload's GEMM times tA * tB)."""
    a, sa = requant_nvfp4_e2m3(w["A"], w["sA"], w["K"])
    b, sb = requant_nvfp4_e2m3(w["B"], w["sB"], w["K"])
    return {"fmt": "mxfp8", "M": w["M"], "N": w["N"], "K": w["K"], "elemA": "e2m3", "elemB": "e2m3",
            "A": a, "sA": sa, "B": b, "sB": sb}


def nvfp4_fp8_workload(w: dict) -> dict:
    """The MXFP8 workload the FP8-rate NVFP4 GEMM computes for NVFP4 workload
    w (its D is this workload's GEMM times tA * tB)."""
    a, sa = requant_nvfp4_mx8(w["A"], w["sA"], w["K"])
    b, sb = requant_nvfp4_mx8(w["B"], w["sB"], w["K"])
    return {"fmt": "mxfp8", "M": w["M"], "N": w["N"], "K": w["K"], "A": a, "sA": sa, "B": b, "sB": sb}


# ---- comparison ------------------------------------------------------------

def rel_errors(d_gpu: np.ndarray, d_ref: np.ndarray, anorm: np.ndarray, bnorm: np.ndarray) -> np.ndarray:
    """r = |D_gpu - D_ref| / max(||dA_m|| ||dB_n|| |alpha|, 2^-1000) per entry;
    non-finite GPU values give r = inf."""
    g = np.asarray(d_gpu, np.float64)
    den = np.maximum(anorm * bnorm, 2.0 ** -1000)
    r = np.abs(g - d_ref) / den
    r[~np.isfinite(g)] = np.inf
    return r
