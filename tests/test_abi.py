"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/dbs.h declares, and rejects bad arguments with a status code before
any device work.  No compute call is made."""
import ctypes
import re
from pathlib import Path

import pytest
import torch

import dense_block_scaled_amd as dbs

ROOT = Path(__file__).resolve().parent.parent


def _declared():
    text = (ROOT / "include" / "dbs.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("gemm_bf16", "gemm_mx", "gemm_mx_mixed", "gemm_nvfp4", "gemm_nvfp4_fp8", "gemm_nvfp4_fp8_workspace",
              "dbs_status_str", "dbs_last_error", "dbs_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = dbs.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.dbs_version() == 102


def test_poison_library_exports_the_same_symbols():
    """The LDS-poison debug build (race-detection tests) is the same library,
    and switching to it and back restores the product build."""
    P = dbs.load_poison_library()
    assert P._name != dbs.lib()._name
    for name in _declared():
        assert hasattr(P, name), name
    assert P.dbs_version() == dbs.lib().dbs_version()
    prod = dbs.lib()
    with dbs.using_library(P):
        assert dbs.lib() is P
    assert dbs.lib() is prod


def test_status_strings():
    for st in (0, 1, 2, 3):
        assert dbs.status_str(st).startswith("DBS_")


FAKE = ctypes.c_void_p(1 << 20)      # 16-byte aligned, never dereferenced
NUL = ctypes.c_void_p(0)


@pytest.mark.parametrize("args,want", [
    ((NUL, FAKE, FAKE, 16, 16, 16, 0, 0), 1),          # null A
    ((FAKE, FAKE, FAKE, 0, 16, 16, 0, 0), 1),          # M = 0
    ((FAKE, FAKE, FAKE, 16, -1, 16, 0, 0), 1),         # N < 0
    ((FAKE, FAKE, FAKE, 16, 16, 12, 0, 0), 1),         # K % 8
    ((FAKE, FAKE, FAKE, 16, 16, 1 << 22, 0, 0), 1),    # K too large
    ((ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, 16, 16, 16, 0, 0), 1),  # misaligned A
    ((FAKE, FAKE, FAKE, 12, 16, 16, 1, 0), 2),         # MN-major A, K-rows of 24 bytes
    ((FAKE, FAKE, FAKE, 16, 20, 16, 0, 1), 2),         # MN-major B, K-rows of 40 bytes
    ((FAKE, FAKE, FAKE, 1 << 16, 16, 1 << 14, 1, 0), 2),  # MN-major A of 2 GiB
    ((FAKE, FAKE, FAKE, 16, 16, 16, 0, 7), 1),         # unknown layout
])
def test_bf16_validation(args, want):
    L = dbs.lib()
    assert L.gemm_bf16(*args, NUL) == want
    assert L.dbs_last_error().decode() != ""


@pytest.mark.parametrize("args,want", [
    ((NUL, FAKE, FAKE, 16, 16, 128, 1), 1),            # null A
    ((FAKE, FAKE, FAKE, 16, 16, 132, 1), 1),           # K % 8
    ((FAKE, FAKE, FAKE, 16, 16, 64, 0), 2),            # one stage: not this kernel
    ((FAKE, FAKE, FAKE, 16, 16, 128, 2), 1),           # release flag not 0 or 1
    ((ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, 16, 16, 128, 1), 1),  # misaligned A
])
def test_bf16_decoupled_validation(args, want):
    L = dbs.lib()
    assert L.gemm_bf16_decoupled(*args, NUL) == want
    assert L.dbs_last_error().decode() != ""


@pytest.mark.parametrize("elem,K,want", [(0, 48, 1), (4, 16, 1), (9, 64, 1), (0, 64, 2)])
def test_mx_validation(elem, K, want):
    L = dbs.lib()
    lb = 1 if want == 2 else 0
    assert L.gemm_mx(elem, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, K, 0, lb, NUL) == want


@pytest.mark.parametrize("ea,eb,lay,want", [
    (0, 4, (1, 0), 2),          # E4M3 x E2M1 MN-major with K % 256 != 0: not implemented
    (4, 1, (0, 1), 2),          # E2M1 x E5M2 MN-major
    (1, 1, (1, 0), 2),          # E5M2 MN-major, M * 8 bits not whole 16-byte K-rows (M = 40)
    (2, 4, (0, 0), 2),          # E2M3 x E2M1: not implemented
    (4, 3, (0, 0), 2),
    (2, 0, (1, 0), 2),          # FP6 MN-major: not implemented
    (0, 3, (0, 1), 2),
    (5, 0, (0, 0), 1),          # unknown element code
    (1, 7, (0, 0), 1),
])
def test_mx_mixed_validation(ea, eb, lay, want):
    L = dbs.lib()
    M = 40 if (ea, eb) == (1, 1) else 64
    assert L.gemm_mx_mixed(ea, eb, FAKE, FAKE, FAKE, FAKE, FAKE, M, 64, 64, *lay, NUL) == want


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would reach a real device")
@pytest.mark.parametrize("ea,eb,lay,K", [(1, 1, (1, 0), 64), (0, 1, (0, 1), 64), (1, 0, (1, 1), 64),
                                         (0, 4, (1, 1), 256), (4, 1, (1, 0), 512)])
def test_mn_major_pairs_pass_validation(ea, eb, lay, K):
    """E5M2 pairs, and FP8 x FP4 pairs with K % 256 == 0, take MN-major
    operands (to the device lookup, which fails here without a GPU)."""
    L = dbs.lib()
    assert L.gemm_mx_mixed(ea, eb, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, K, *lay, NUL) == 3


def test_fp4_mn_rows_need_32_elements():
    """An MN-major E2M1 operand beside an 8-bit one needs M (or N) a multiple
    of 32 (whole 16-byte K-rows); the 8-bit one a multiple of 16."""
    L = dbs.lib()
    assert L.gemm_mx_mixed(4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 48, 64, 256, 1, 0, NUL) == 2
    assert L.gemm_mx_mixed(0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 48, 256, 0, 1, NUL) == 2
    assert L.dbs_last_error().decode() != ""


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would reach a real device")
@pytest.mark.parametrize("ea,eb", [(0, 1), (1, 0), (1, 1), (4, 4), (0, 4), (4, 0), (1, 4), (4, 1)])
def test_mx_mixed_valid_pairs_pass_validation(ea, eb):
    L = dbs.lib()
    assert L.gemm_mx_mixed(ea, eb, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 0, 0, NUL) == 3
    assert L.gemm_mx(1, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 0, 0, NUL) == 3


def test_nvfp4_fp8_workspace_size():
    L = dbs.lib()
    L.gemm_nvfp4_fp8_workspace.restype = ctypes.c_size_t
    L.gemm_nvfp4_fp8_workspace.argtypes = [ctypes.c_int64] * 3
    a256 = lambda x: -(-x // 256) * 256
    assert L.gemm_nvfp4_fp8_workspace(300, 200, 64) == a256(300 * 64) + a256(200 * 64) + a256(300 * 2) + a256(200 * 2)
    assert L.gemm_nvfp4_fp8_workspace(300, 200, 48) == 0          # K % 32
    assert L.gemm_nvfp4_fp8_workspace(0, 200, 64) == 0


@pytest.mark.parametrize("K,ws,nbytes,lay,want", [
    (48, FAKE, 1 << 30, (0, 0), 2),                       # K % 32 == 16: not implemented
    (40, FAKE, 1 << 30, (0, 0), 1),                       # K % 16
    (64, NUL, 1 << 30, (0, 0), 1),                        # no workspace
    (64, ctypes.c_void_p((1 << 20) + 16), 1 << 30, (0, 0), 1),   # workspace not 256-byte aligned
    (64, FAKE, 100, (0, 0), 1),                           # workspace too small
    (64, FAKE, 1 << 30, (1, 0), 2),                       # MN-major
])
def test_nvfp4_fp8_validation(K, ws, nbytes, lay, want):
    L = dbs.lib()
    st = L.gemm_nvfp4_fp8(FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE, ctypes.c_float(1.0), FAKE, 64, 64, K, *lay,
                          ws, ctypes.c_size_t(nbytes), NUL)
    assert st == want, dbs.status_str(st)


def test_mx_null_scales():
    L = dbs.lib()
    assert L.gemm_mx(0, FAKE, NUL, FAKE, FAKE, FAKE, 8, 8, 64, 0, 0, NUL) == 1


@pytest.mark.parametrize("M,K,lay,want", [
    (64, 24, (0, 0), 1), (64, 40, (0, 0), 1),
    (64, 48, (1, 0), 2), (64, 48, (0, 1), 2),          # K-major beside MN-major: K % 32 == 0 only
    (48, 64, (1, 0), 2),                               # MN-major A: M * 4 bits not whole 16-byte rows
])
def test_nvfp4_validation(M, K, lay, want):
    L = dbs.lib()
    assert L.gemm_nvfp4(FAKE, FAKE, 1.0, FAKE, FAKE, 1.0, FAKE, M, 64, K, *lay, NUL) == want


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would reach a real device")
@pytest.mark.parametrize("fmt,M,N,K,lay", [("bf16", 8, 24, 64, (1, 1)), ("e4m3", 16, 48, 64, (1, 0)),
                                            ("e2m1", 64, 32, 64, (0, 1)), ("nvfp4", 8, 8, 48, (0, 0)),
                                            ("nvfp4", 8, 8, 16, (0, 0)), ("nvfp4", 32, 64, 48, (1, 1)),
                                            ("nvfp4", 32, 8, 64, (1, 0)), ("nvfp4", 8, 32, 64, (0, 1))])
def test_valid_requests_pass_validation(fmt, M, N, K, lay):
    """MN-major operands with whole 16-byte K-rows, and NVFP4 with K an odd
    multiple of 16 (with both operands MN-major, or both K-major), get past
    validation (to the device lookup, which fails here without a GPU)."""
    L = dbs.lib()
    if fmt == "bf16":
        st = L.gemm_bf16(FAKE, FAKE, FAKE, M, N, K, *lay, NUL)
    elif fmt == "nvfp4":
        st = L.gemm_nvfp4(FAKE, FAKE, 1.0, FAKE, FAKE, 1.0, FAKE, M, N, K, *lay, NUL)
    else:
        st = L.gemm_mx(0 if fmt == "e4m3" else 4, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, *lay, NUL)
    assert st == 3, dbs.status_str(st)


def test_binding_layout_shapes():
    """The binding reads M, N and K from MN-major shapes and checks them."""
    A = torch.zeros((32, 8), dtype=torch.bfloat16)          # MN-major: K = 32, M = 8
    B = torch.zeros((24, 32), dtype=torch.bfloat16)         # K-major: N = 24
    with pytest.raises(ValueError, match="GPU tensor"):
        dbs.gemm_bf16(A, B, la=dbs.MN_MAJOR)
    with pytest.raises(ValueError, match="layout"):
        dbs.gemm_bf16(A, B, la=5)
    assert dbs._shape(8, 32, dbs.MN_MAJOR) == (32, 8)
    assert dbs._shape(64, 32, dbs.MN_MAJOR, 2) == (32, 32)
    assert dbs._rows(torch.zeros((32, 16), dtype=torch.uint8), dbs.MN_MAJOR, 2) == 32


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would reach a real device")
def test_no_device_reports_ehip_without_aborting():
    L = dbs.lib()
    st = L.gemm_bf16(FAKE, FAKE, FAKE, 16, 16, 16, 0, 0, NUL)
    assert st == 3
    assert L.dbs_last_error().decode()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(dbs, "_lib", None)
    monkeypatch.setattr(dbs, "LIB_PATH", tmp_path / "libdbs.so")
    with pytest.raises(ImportError):
        dbs.lib()


def test_binding_rejects_cpu_tensors():
    A = torch.zeros((8, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dbs.gemm_bf16(A, A)


# ---- quantisers ----------------------------------------------------------------

@pytest.mark.parametrize("elem,x,codes,scales,K,want", [
    (0, FAKE, FAKE, FAKE, 48, 1),                               # K % 32
    (9, FAKE, FAKE, FAKE, 64, 1),                               # unknown element format
    (0, NUL, FAKE, FAKE, 64, 1),                                # null x
    (4, FAKE, FAKE, NUL, 64, 1),                                # null scales
    (0, ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, 64, 1),     # misaligned x
    (4, FAKE, ctypes.c_void_p((1 << 20) + 8), FAKE, 64, 1),     # misaligned codes
])
def test_quant_mx_validation(elem, x, codes, scales, K, want):
    L = dbs.lib()
    assert L.quant_mx(elem, x, 4, K, codes, scales, NUL) == want
    assert L.dbs_last_error().decode() != ""


@pytest.mark.parametrize("K,t,rows,want", [(24, FAKE, 4, 1), (32, NUL, 4, 1), (32, FAKE, 0, 1)])
def test_quant_nvfp4_validation(K, t, rows, want):
    L = dbs.lib()
    assert L.quant_nvfp4(FAKE, rows, K, FAKE, FAKE, t, NUL) == want


@pytest.mark.parametrize("n,want", [(12, 1), (0, 1)])
def test_quant_bf16_validation(n, want):
    L = dbs.lib()
    assert L.quant_bf16(FAKE, n, FAKE, NUL) == want


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would reach a real device")
def test_quant_no_device_reports_ehip():
    L = dbs.lib()
    assert L.quant_mx(0, FAKE, 4, 64, FAKE, FAKE, NUL) == 3


def test_quant_binding_rejects_cpu_tensors():
    with pytest.raises(ValueError):
        dbs.quant_mx("e4m3", torch.zeros((4, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        dbs.quant_nvfp4(torch.zeros((4, 64), dtype=torch.float32))


# ---- grouped GEMMs -------------------------------------------------------------------

def _off(*v):
    return (ctypes.c_int64 * len(v))(*v)


@pytest.mark.parametrize("off,G,want", [
    (_off(0, 8, 16), 2, None),          # valid (reaches the device check)
    (_off(1, 8, 16), 2, 1),             # offsets[0] != 0
    (_off(0, 9, 4), 2, 1),              # decreasing
    (_off(0, 0, 0), 2, 1),              # no rows at all
    (_off(0, 8), 0, 1),                 # G < 1
    (_off(*range(0, 66)), 65, 1),       # G > 64
])
def test_grouped_validation(off, G, want):
    L = dbs.lib()
    st = L.gemm_grouped_bf16(FAKE, FAKE, FAKE, off, G, 16, 16, NUL)
    if want is None:
        assert st in (0, 3)             # 3: no device here
    else:
        assert st == want


def test_grouped_null_arguments():
    L = dbs.lib()
    assert L.gemm_grouped_bf16(FAKE, FAKE, FAKE, NUL, 2, 16, 16, NUL) == 1
    assert L.gemm_grouped_mx(0, FAKE, NUL, FAKE, FAKE, FAKE, _off(0, 8, 16), 2, 16, 64, NUL) == 1
    assert L.gemm_grouped_nvfp4(FAKE, FAKE, 1.0, FAKE, FAKE, NUL, FAKE, _off(0, 8, 16), 2, 16, 64, NUL) == 1
    assert L.gemm_grouped_mx(0, FAKE, FAKE, FAKE, FAKE, FAKE, _off(0, 8, 16), 2, 16, 48, NUL) == 1   # K % 32


def test_nvfp4_fp8_noalloc_validation():
    """The allocation-free FP8-rate entry point validates like gemm_nvfp4_fp8,
    rejects problems whose workspace exceeds its static 64 MiB before any
    device work, and reports the missing device on a valid small problem."""
    L = dbs.lib()
    f = ctypes.c_float(1.0)
    call = lambda M, N, K, la=0: L.gemm_nvfp4_fp8_noalloc(FAKE, FAKE, f, FAKE, FAKE, f, FAKE, M, N, K, la, 0, NUL)
    assert call(64, 64, 48) == 2                                 # K % 32 != 0
    assert call(64, 64, 64, la=1) == 2                           # MN-major
    assert call(0, 64, 64) == 1
    assert L.gemm_nvfp4_fp8_workspace(4096, 4096, 8192) > (64 << 20)
    assert call(4096, 4096, 8192) == 1
    assert "workspace" in L.dbs_last_error().decode()
    assert call(256, 256, 256) == 3                              # no GPU here


def test_nvfp4_fp6_workspace_and_validation():
    """The FP4-rate NVFP4 entry point: workspace size (E2M3 codes of both
    operands, 3K/4 bytes per row with the rows padded to a multiple of 8,
    and their E8M0 scales, each part 256-byte aligned), validation before
    any device work."""
    L = dbs.lib()
    a256 = lambda x: (x + 255) // 256 * 256
    r8 = lambda x: (x + 7) // 8 * 8
    for M, N, K in [(300, 200, 512), (301, 203, 512), (1, 9, 96)]:
        want = a256(r8(M) * K * 3 // 4) + a256(r8(N) * K * 3 // 4) + a256(M * K // 32) + a256(N * K // 32)
        assert L.gemm_nvfp4_fp6_workspace(M, N, K) == want, (M, N, K)
    assert L.gemm_nvfp4_fp6_workspace(M, N, 48) == 0
    f = ctypes.c_float(1.0)
    call = lambda M, N, K, ws, nb, la=0: L.gemm_nvfp4_fp6(FAKE, FAKE, f, FAKE, FAKE, f, FAKE, M, N, K, la, 0, ws, nb,
                                                          NUL)
    assert call(64, 64, 64, NUL, 1 << 20) == 1                   # no workspace
    assert call(64, 64, 48, FAKE, 1 << 20) == 2                  # K % 32
    assert call(64, 64, 64, FAKE, 1 << 20, la=1) == 2            # MN-major
    assert call(64, 64, 64, ctypes.c_void_p((1 << 20) + 64), 1 << 20) == 1   # misaligned workspace
    assert call(64, 64, 64, FAKE, 16) == 1                       # too small
    assert call(64, 64, 64, FAKE, 1 << 20) == 3                  # no GPU here
