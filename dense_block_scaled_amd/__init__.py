"""MI355X (gfx950) block-scaled GEMM: thin Python binding of libdbs.so.

    D = bf16(alpha * (sA . A) @ (sB . B)^T),  fp32 accumulation

The functions take torch tensors that already live on the GPU and only
marshal pointers, sizes and the current stream into the C ABI of
``include/dbs.h``; every step of the computation runs in the HIP kernels.
There is no CPU fallback: if ``libdbs.so`` is missing, or a call reports an
error, these functions raise.

Operand encodings (contiguous; K-major unless la / lb say MN_MAJOR):
  gemm_bf16(A, B)                     A: (M, K) bfloat16/uint16, B: (N, K)
  gemm_bf16_decoupled(A, B)           the same on the decoupled-ring kernel (K-major, K > 64)
  gemm_mx(elem, A, sA, B, sB)         elem 'e4m3': A (M, K) uint8;
                                      elem 'e2m1': A (M, K/2) uint8, 2 per byte
                                      sA: (M, K/32) uint8 E8M0 codes
  gemm_nvfp4(A, sA, tA, B, sB, tB)    A: (M, K/2) uint8 packed E2M1,
                                      sA: (M, K/16) uint8 E4M3 codes, tA float
MN-major operands (gemm_bf16, gemm_mx) are stored transposed: A (K, M), B
(K, N), E2M1 packing two consecutive M (N) per byte, (K, M/2); scales keep
their (M, K/32) layout.
Each returns D: (M, N) torch.bfloat16 (or writes into ``out``).
"""
from __future__ import annotations

import contextlib
import ctypes
from pathlib import Path

import torch

__all__ = ["gemm_bf16", "gemm_bf16_decoupled", "gemm_mx", "gemm_mx_mixed", "gemm_nvfp4", "gemm_nvfp4_fp8", "gemm_nvfp4_fp8_noalloc", "nvfp4_fp8_workspace_bytes", "gemm_nvfp4_fp6", "nvfp4_fp6_workspace_bytes", "gemm_grouped_bf16", "gemm_grouped_mx", "gemm_grouped_nvfp4", "quant_mx", "quant_nvfp4", "quant_bf16", "lib", "LIB_PATH", "DbsError", "load_poison_library", "using_library",
           "DBS_OK", "DBS_EINVAL", "DBS_EUNSUPPORTED", "DBS_EHIP", "K_MAJOR", "MN_MAJOR",
           "E4M3", "E5M2", "E2M3", "E3M2", "E2M1", "status_str"]

LIB_PATH = Path(__file__).resolve().parent / "libdbs.so"

DBS_OK, DBS_EINVAL, DBS_EUNSUPPORTED, DBS_EHIP = 0, 1, 2, 3
K_MAJOR, MN_MAJOR = 0, 1
E4M3, E5M2, E2M3, E3M2, E2M1 = 0, 1, 2, 3, 4
_ELEM = {"e4m3": E4M3, "e5m2": E5M2, "e2m3": E2M3, "e3m2": E3M2, "e2m1": E2M1}


class DbsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def _load(path: Path) -> ctypes.CDLL:
    if not path.exists():
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m dense_block_scaled_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(str(path))
    _declare(L)
    return L


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def load_poison_library() -> ctypes.CDLL:
    """The LDS-poison debug build of the library (libdbs_poison.so: every
    direct-to-LDS load first fills its destination with 0xFF), for the
    race-detection tests; raises if it has not been built."""
    return _load(LIB_PATH.with_name("libdbs_poison.so"))


@contextlib.contextmanager
def using_library(L: ctypes.CDLL):
    """Route this module's calls through library L (e.g. the poison build)
    inside the block."""
    global _lib
    prev = lib()
    _lib = L
    try:
        yield L
    finally:
        _lib = prev


def _declare(L: ctypes.CDLL) -> None:
    """Argument and result types of the C ABI's entry points."""
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.gemm_bf16.argtypes = [P, P, P, I64, I64, I64, I, I, P]
    L.gemm_bf16.restype = I
    L.gemm_bf16_decoupled.argtypes = [P, P, P, I64, I64, I64, I, P]
    L.gemm_bf16_decoupled.restype = I
    L.gemm_mx.argtypes = [I, P, P, P, P, P, I64, I64, I64, I, I, P]
    L.gemm_mx.restype = I
    L.gemm_mx_mixed.argtypes = [I, I, P, P, P, P, P, I64, I64, I64, I, I, P]
    L.gemm_mx_mixed.restype = I
    L.gemm_nvfp4.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, P, I64, I64, I64, I, I, P]
    L.gemm_nvfp4.restype = I
    L.gemm_nvfp4_fp8_workspace.argtypes = [I64, I64, I64]
    L.gemm_nvfp4_fp8_workspace.restype = ctypes.c_size_t
    L.gemm_nvfp4_fp8.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, P, I64, I64, I64, I, I, P,
                                 ctypes.c_size_t, P]
    L.gemm_nvfp4_fp8.restype = I
    L.gemm_nvfp4_fp6_workspace.argtypes = [I64, I64, I64]
    L.gemm_nvfp4_fp6_workspace.restype = ctypes.c_size_t
    L.gemm_nvfp4_fp6.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, P, I64, I64, I64, I, I, P,
                                 ctypes.c_size_t, P]
    L.gemm_nvfp4_fp6.restype = I
    L.gemm_nvfp4_fp8_noalloc.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, P, I64, I64, I64, I, I, P]
    L.gemm_nvfp4_fp8_noalloc.restype = I
    L.gemm_grouped_bf16.argtypes = [P, P, P, P, I64, I64, I64, P]
    L.gemm_grouped_bf16.restype = I
    L.gemm_grouped_mx.argtypes = [I, P, P, P, P, P, P, I64, I64, I64, P]
    L.gemm_grouped_mx.restype = I
    L.gemm_grouped_nvfp4.argtypes = [P, P, ctypes.c_float, P, P, P, P, P, I64, I64, I64, P]
    L.gemm_grouped_nvfp4.restype = I
    L.quant_mx.argtypes = [I, P, I64, I64, P, P, P]
    L.quant_mx.restype = I
    L.quant_nvfp4.argtypes = [P, I64, I64, P, P, P, P]
    L.quant_nvfp4.restype = I
    L.quant_bf16.argtypes = [P, I64, P, P]
    L.quant_bf16.restype = I
    L.dbs_status_str.argtypes = [I]
    L.dbs_status_str.restype = ctypes.c_char_p
    L.dbs_last_error.argtypes = []
    L.dbs_last_error.restype = ctypes.c_char_p
    L.dbs_version.restype = I


def status_str(st: int) -> str:
    return lib().dbs_status_str(st).decode()


def _check(st: int) -> None:
    if st != DBS_OK:
        raise DbsError(st, f"{status_str(st)}: {lib().dbs_last_error().decode()}")


def _dev(t: torch.Tensor, name: str, dtypes, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _out(out, M, N, like):
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=like.device)
    _dev(out, "out", (torch.bfloat16, torch.int16, torch.uint16), (M, N))
    return out


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _layout(l: int, name: str) -> int:
    if l not in (K_MAJOR, MN_MAJOR):
        raise ValueError(f"{name}: layout must be K_MAJOR or MN_MAJOR")
    return l


def _rows(t: torch.Tensor, l: int, per_byte: int = 1) -> int:
    """M (or N) of an operand: its row count, or (MN-major) its columns."""
    return t.shape[0] if l == K_MAJOR else t.shape[1] * per_byte


def _shape(rows: int, kcols: int, l: int, per_byte: int = 1) -> tuple:
    """Expected tensor shape of an operand with `rows` rows (M or N) and K
    of kcols elements (per_byte elements per stored byte)."""
    return (rows, kcols // per_byte) if l == K_MAJOR else (kcols, rows // per_byte)


def gemm_bf16(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None,
              la: int = K_MAJOR, lb: int = K_MAJOR) -> torch.Tensor:
    """D = A @ B^T for bf16 A (M, K), B (N, K) (MN-major: (K, M), (K, N));
    fp32 accumulate, bf16 out."""
    la, lb = _layout(la, "la"), _layout(lb, "lb")
    M, N = _rows(A, la), _rows(B, lb)
    K = A.shape[1] if la == K_MAJOR else A.shape[0]
    dt = (torch.bfloat16, torch.int16, torch.uint16)
    pa = _dev(A, "A", dt, _shape(M, K, la))
    pb = _dev(B, "B", dt, _shape(N, K, lb))
    out = _out(out, M, N, A)
    _check(lib().gemm_bf16(pa, pb, ctypes.c_void_p(out.data_ptr()), M, N, K, la, lb, _stream(A)))
    return out


def gemm_bf16_decoupled(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None,
                        early_release_a: bool = True) -> torch.Tensor:
    """gemm_bf16 (K-major A (M, K), B (N, K)) on the kernel with decoupled A
    and B rings, A's slot released early (or at the stage's end); K > 64."""
    M, K = A.shape
    N = B.shape[0]
    dt = (torch.bfloat16, torch.int16, torch.uint16)
    pa = _dev(A, "A", dt, (M, K))
    pb = _dev(B, "B", dt, (N, K))
    out = _out(out, M, N, A)
    _check(lib().gemm_bf16_decoupled(pa, pb, ctypes.c_void_p(out.data_ptr()), M, N, K, int(bool(early_release_a)),
                                     _stream(A)))
    return out


def gemm_mx(elem: str, A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor,
            K: int | None = None, out: torch.Tensor | None = None,
            la: int = K_MAJOR, lb: int = K_MAJOR) -> torch.Tensor:
    """MXFP8 (elem='e4m3' or 'e5m2'), MXFP6 (elem='e2m3' or 'e3m2', K-major)
    or MXFP4 (elem='e2m1') GEMM with E8M0 scales per 32."""
    return gemm_mx_mixed(elem, elem, A, sA, B, sB, K=K, out=out, la=la, lb=lb)


def gemm_mx_mixed(elem_a: str, elem_b: str, A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor,
                  sB: torch.Tensor, K: int | None = None, out: torch.Tensor | None = None,
                  la: int = K_MAJOR, lb: int = K_MAJOR) -> torch.Tensor:
    """MX GEMM with A's elements in elem_a and B's in elem_b ('e4m3', 'e5m2',
    'e2m1', or the FP6 'e2m3' / 'e3m2', four elements per three bytes; the
    library takes every pairing except FP6 with E2M1, FP6 K-major only)."""
    code_a, code_b = _ELEM[elem_a], _ELEM[elem_b]
    la, lb = _layout(la, "la"), _layout(lb, "lb")
    fp6 = ("e2m3", "e3m2")
    if (elem_a in fp6 and la != K_MAJOR) or (elem_b in fp6 and lb != K_MAJOR):
        raise ValueError("FP6 operands are K-major only")
    pa_ = 2 if elem_a == "e2m1" else 1   # elements per byte (FP6: 4 per 3, K-major)
    pb_ = 2 if elem_b == "e2m1" else 1
    M, N = _rows(A, la, pa_), _rows(B, lb, pb_)
    if K is None:
        K = (A.shape[1] * 4 // 3 if elem_a in fp6 else A.shape[1] * pa_) if la == K_MAJOR else A.shape[0]
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, (M, K // 4 * 3) if elem_a in fp6 else _shape(M, K, la, pa_))
    pb = _dev(B, "B", u8, (N, K // 4 * 3) if elem_b in fp6 else _shape(N, K, lb, pb_))
    psa = _dev(sA, "sA", u8, (M, K // 32))
    psb = _dev(sB, "sB", u8, (N, K // 32))
    out = _out(out, M, N, A)
    _check(lib().gemm_mx_mixed(code_a, code_b, pa, psa, pb, psb, ctypes.c_void_p(out.data_ptr()), M, N, K,
                               la, lb, _stream(A)))
    return out


def gemm_nvfp4(A: torch.Tensor, sA: torch.Tensor, tA: float, B: torch.Tensor, sB: torch.Tensor, tB: float,
               out: torch.Tensor | None = None, la: int = K_MAJOR, lb: int = K_MAJOR) -> torch.Tensor:
    """NVFP4 GEMM: packed E2M1 with E4M3 scales per 16 and fp32 tensor scales
    (MN-major operands: (K, M / 2), (K, N / 2) bytes; scales stay (rows, K / 16))."""
    la, lb = _layout(la, "la"), _layout(lb, "lb")
    M, N = _rows(A, la, 2), _rows(B, lb, 2)
    K = A.shape[1] * 2 if la == K_MAJOR else A.shape[0]
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, _shape(M, K, la, 2))
    pb = _dev(B, "B", u8, _shape(N, K, lb, 2))
    psa = _dev(sA, "sA", u8, (M, K // 16))
    psb = _dev(sB, "sB", u8, (N, K // 16))
    out = _out(out, M, N, A)
    _check(lib().gemm_nvfp4(pa, psa, float(tA), pb, psb, float(tB), ctypes.c_void_p(out.data_ptr()),
                            M, N, K, la, lb, _stream(A)))
    return out


def nvfp4_fp8_workspace_bytes(M: int, N: int, K: int) -> int:
    """Device workspace gemm_nvfp4_fp8 needs for an M x N x K problem (0 if
    the sizes are invalid)."""
    return int(lib().gemm_nvfp4_fp8_workspace(M, N, K))


def gemm_nvfp4_fp8(A: torch.Tensor, sA: torch.Tensor, tA: float, B: torch.Tensor, sB: torch.Tensor, tB: float,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """FP8-rate NVFP4 GEMM (opt-in, lossy; see include/dbs.h): the NVFP4
    operands of gemm_nvfp4 are requantised to MXFP8 in ``workspace`` (a uint8
    GPU tensor of at least nvfp4_fp8_workspace_bytes(M, N, K) bytes, allocated
    here if not given) and multiplied at the 8-bit MFMA rate."""
    M, N = A.shape[0], B.shape[0]
    K = A.shape[1] * 2
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, (M, K // 2))
    pb = _dev(B, "B", u8, (N, K // 2))
    psa = _dev(sA, "sA", u8, (M, K // 16))
    psb = _dev(sB, "sB", u8, (N, K // 16))
    out = _out(out, M, N, A)
    need = nvfp4_fp8_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=A.device)
    _dev(workspace, "workspace", u8, (workspace.numel(),))
    _check(lib().gemm_nvfp4_fp8(pa, psa, float(tA), pb, psb, float(tB), ctypes.c_void_p(out.data_ptr()),
                                M, N, K, K_MAJOR, K_MAJOR, ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel(), _stream(A)))
    return out


# ---- quantisers (fp32 -> GEMM input formats, on the GPU) ----------------------

def quant_mx(elem: str, x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """fp32 x (rows, K) -> (codes, E8M0 scales per 32): codes (rows, K) uint8
    for elem='e4m3' or 'e5m2', (rows, K/2) packed for elem='e2m1', (rows,
    3K/4) packed for the FP6 'e2m3' / 'e3m2'; scales (rows, K/32)."""
    code = _ELEM[elem]
    rows, K = x.shape
    px = _dev(x, "x", (torch.float32,), (rows, K))
    width = {"e2m1": K // 2, "e2m3": K // 4 * 3, "e3m2": K // 4 * 3}.get(elem, K)
    codes = torch.empty((rows, width), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().quant_mx(code, px, rows, K, ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                          _stream(x)))
    return codes, scales


def quant_nvfp4(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """fp32 x (rows, K) -> (packed E2M1 codes (rows, K/2), E4M3 scales per 16
    (rows, K/16), tensor scale t as a one-element fp32 GPU tensor)."""
    rows, K = x.shape
    px = _dev(x, "x", (torch.float32,), (rows, K))
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=x.device)
    t = torch.empty((1,), dtype=torch.float32, device=x.device)
    _check(lib().quant_nvfp4(px, rows, K, ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                             ctypes.c_void_p(t.data_ptr()), _stream(x)))
    return codes, scales, t


def quant_bf16(x: torch.Tensor) -> torch.Tensor:
    """fp32 x -> bf16 (round to nearest even), same shape."""
    px = _dev(x, "x", (torch.float32,), tuple(x.shape))
    out = torch.empty(tuple(x.shape), dtype=torch.bfloat16, device=x.device)
    _check(lib().quant_bf16(px, x.numel(), ctypes.c_void_p(out.data_ptr()), _stream(x)))
    return out


# ---- grouped GEMMs (mixture-of-experts layout) ----------------------------------

def _offsets(offsets) -> tuple[ctypes.Array, int]:
    off = [int(v) for v in offsets]
    return (ctypes.c_int64 * len(off))(*off), len(off) - 1


def gemm_grouped_bf16(A: torch.Tensor, B: torch.Tensor, offsets, out: torch.Tensor | None = None) -> torch.Tensor:
    """Group g: D[off[g]:off[g+1]] = A[off[g]:off[g+1]] @ B[g]^T; A (M, K) and
    B (G, N, K) bf16, offsets a host sequence of G + 1 row offsets."""
    off, G = _offsets(offsets)
    M, K = A.shape
    N = B.shape[1]
    dt = (torch.bfloat16, torch.int16, torch.uint16)
    pa = _dev(A, "A", dt, (M, K))
    pb = _dev(B, "B", dt, (G, N, K))
    out = _out(out, M, N, A)
    _check(lib().gemm_grouped_bf16(pa, pb, ctypes.c_void_p(out.data_ptr()), off, G, N, K, _stream(A)))
    return out


def gemm_grouped_mx(elem: str, A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor, offsets,
                    K: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped MXFP8 / MXFP4 GEMM: A (M, K bytes) with sA (M, K/32); B (G, N, K
    bytes) with sB (G, N, K/32); offsets as for gemm_grouped_bf16."""
    code = _ELEM[elem]
    off, G = _offsets(offsets)
    M, N = A.shape[0], B.shape[1]
    if K is None:
        K = A.shape[1] * (2 if elem == "e2m1" else 1)
    kb = K // 2 if elem == "e2m1" else K
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, (M, kb))
    pb = _dev(B, "B", u8, (G, N, kb))
    psa = _dev(sA, "sA", u8, (M, K // 32))
    psb = _dev(sB, "sB", u8, (G, N, K // 32))
    out = _out(out, M, N, A)
    _check(lib().gemm_grouped_mx(code, pa, psa, pb, psb, ctypes.c_void_p(out.data_ptr()), off, G, N, K, _stream(A)))
    return out


def gemm_grouped_nvfp4(A: torch.Tensor, sA: torch.Tensor, tA: float, B: torch.Tensor, sB: torch.Tensor, tB,
                       offsets, out: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped NVFP4 GEMM: one tensor scale tA for A, one tB[g] per group of B."""
    off, G = _offsets(offsets)
    M, N = A.shape[0], B.shape[1]
    K = A.shape[1] * 2
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, (M, K // 2))
    pb = _dev(B, "B", u8, (G, N, K // 2))
    psa = _dev(sA, "sA", u8, (M, K // 16))
    psb = _dev(sB, "sB", u8, (G, N, K // 16))
    tb = (ctypes.c_float * G)(*[float(v) for v in tB])
    out = _out(out, M, N, A)
    _check(lib().gemm_grouped_nvfp4(pa, psa, float(tA), pb, psb, tb, ctypes.c_void_p(out.data_ptr()), off, G, N, K,
                                    _stream(A)))
    return out


def gemm_nvfp4_fp8_noalloc(A: torch.Tensor, sA: torch.Tensor, tA: float, B: torch.Tensor, sB: torch.Tensor,
                           tB: float, out: torch.Tensor) -> torch.Tensor:
    """gemm_nvfp4_fp8 without any allocation: the library's static 64 MiB
    device workspace replaces the caller's (see include/dbs.h; problems whose
    workspace would be larger raise DbsError with DBS_EINVAL).  ``out`` (M x N
    bfloat16 on the GPU) is required, since allocating it would defeat the
    purpose."""
    M, N = A.shape[0], B.shape[0]
    K = A.shape[1] * 2
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, (M, K // 2))
    pb = _dev(B, "B", u8, (N, K // 2))
    psa = _dev(sA, "sA", u8, (M, K // 16))
    psb = _dev(sB, "sB", u8, (N, K // 16))
    po = _dev(out, "out", (torch.bfloat16,), (M, N))
    _check(lib().gemm_nvfp4_fp8_noalloc(pa, psa, float(tA), pb, psb, float(tB), po, M, N, K, K_MAJOR, K_MAJOR,
                                        _stream(A)))
    return out


def nvfp4_fp6_workspace_bytes(M: int, N: int, K: int) -> int:
    """Device workspace gemm_nvfp4_fp6 needs for an M x N x K problem (0 if
    the sizes are invalid)."""
    return int(lib().gemm_nvfp4_fp6_workspace(M, N, K))


def gemm_nvfp4_fp6(A: torch.Tensor, sA: torch.Tensor, tA: float, B: torch.Tensor, sB: torch.Tensor, tB: float,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """FP4-rate NVFP4 GEMM (opt-in, lossy; see include/dbs.h): the NVFP4
    operands are requantised to MXFP6 E2M3 in ``workspace`` (a uint8 GPU
    tensor of at least nvfp4_fp6_workspace_bytes(M, N, K) bytes, allocated
    here if not given) and multiplied at the FP6 (= FP4) MFMA rate."""
    M, N = A.shape[0], B.shape[0]
    K = A.shape[1] * 2
    u8 = (torch.uint8,)
    pa = _dev(A, "A", u8, (M, K // 2))
    pb = _dev(B, "B", u8, (N, K // 2))
    psa = _dev(sA, "sA", u8, (M, K // 16))
    psb = _dev(sB, "sB", u8, (N, K // 16))
    out = _out(out, M, N, A)
    need = nvfp4_fp6_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=A.device)
    _dev(workspace, "workspace", u8, (workspace.numel(),))
    _check(lib().gemm_nvfp4_fp6(pa, psa, float(tA), pb, psb, float(tB), ctypes.c_void_p(out.data_ptr()),
                                M, N, K, K_MAJOR, K_MAJOR, ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel(), _stream(A)))
    return out
