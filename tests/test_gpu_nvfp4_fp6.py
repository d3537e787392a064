"""GPU checks of the opt-in FP4-rate NVFP4 GEMM (gemm_nvfp4_fp6) through the C
ABI: its E2M3 requantised operands bit for bit against the oracle's recipe
(every pair of E4M3 group scales with every E2M1 code), its result against
the oracle GEMM of those operands (the usual parity bar) on both GEMM paths
(the FP6-rate 256 x 256 kernel and the widening path), its distance from the
exact NVFP4 result within the stated bound, and exactness at unit scales."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import oracle
import synth
from tests import _gpu, _pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _a256(x):
    return -(-x // 256) * 256


def run_fp6(w: dict):
    """D and the workspace tensor after the call."""
    d = _gpu.to_dev(w)
    M, N, K = w["M"], w["N"], w["K"]
    ws = torch.empty(dbs.nvfp4_fp6_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    D = dbs.gemm_nvfp4_fp6(d["A"], d["sA"], w["tA"], d["B"], d["sB"], w["tB"], workspace=ws)
    return D, ws


def _r8(x):
    return -(-x // 8) * 8


def fp6_rate(M, N, K):
    """Whether the GEMM runs on the FP6-rate kernel (256 x 256 tiles filling
    at least a quarter of the CUs, K whole 128-K stages), which reads the
    requantised codes stage-blocked."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return K % 128 == 0 and 4 * (-(-M // 256)) * (-(-N // 256)) >= cus


def _unblock(h, rows, K):
    """Row-major rows x 3K/4 codes from the stage-blocked layout: the 96
    bytes of stage ks of rows 8g .. 8g+7 at (g nk + ks) 768 + 96 (row % 8);
    the padding rows (up to a multiple of 8) must hold zero codes."""
    nk = K // 128
    x = h.reshape(_r8(rows) // 8, nk, 8, 96).transpose(0, 2, 1, 3).reshape(_r8(rows), nk * 96)
    assert not x[rows:].any(), "padding rows of the stage-blocked codes are not zero"
    return x[:rows]


def _ws_parts(ws, M, N, K):
    """The workspace's A codes, B codes (row-major, rows x 3K/4), A scales, B
    scales (rows x K/32)."""
    h = ws.cpu().numpy()
    ra, rb = _r8(M) * K // 4 * 3, _r8(N) * K // 4 * 3
    ob = _a256(ra)
    osa = ob + _a256(rb)
    osb = osa + _a256(M * K // 32)
    if fp6_rate(M, N, K):
        a, b = _unblock(h[:ra], M, K), _unblock(h[ob:ob + rb], N, K)
    else:
        a, b = h[:M * K // 4 * 3].reshape(M, K // 4 * 3), h[ob:ob + N * K // 4 * 3].reshape(N, K // 4 * 3)
    return a, b, h[osa:osa + M * K // 32].reshape(M, K // 32), h[osb:osb + N * K // 32].reshape(N, K // 32)


def _r(got, d_ref, an, bn):
    return oracle.rel_errors(got, d_ref, an, bn)


# the FP6-rate kernel (256 x 256 tiles, K % 128 == 0: the first four; the
# third with rows that leave partial groups of 8 and an odd stage count, the
# fourth at exactly a quarter of the CUs' worth of tiles on a 256-CU part),
# the widening path (few tiles; K % 128 != 0)
SHAPES = [(2304, 2304, 512), (2200, 2600, 256), (2301, 2299, 640), (256, 16384, 512), (300, 520, 384),
          (2304, 2304, 352)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_requant_and_gemm(shape):
    M, N, K = shape
    _gpu.say(f"[nvfp4-fp6] {shape}")
    w = synth.workload("nvfp4", M, N, K, 930 + M % 31, 940 + N % 37)
    D, ws = run_fp6(w)
    torch.cuda.synchronize()
    a, b, sa, sb = _ws_parts(ws, M, N, K)
    ra, rsa = oracle.requant_nvfp4_e2m3(w["A"], w["sA"], K)
    rb, rsb = oracle.requant_nvfp4_e2m3(w["B"], w["sB"], K)
    assert np.array_equal(sa, rsa) and np.array_equal(sb, rsb)
    assert np.array_equal(a, ra) and np.array_equal(b, rb)
    wq = oracle.nvfp4_fp6_workload(w)
    alpha = float(np.float32(w["tA"]) * np.float32(w["tB"]))
    em, en = synth.sample_entries(74, M, N, 4096)
    got = _gpu.d_to_numpy(D)[em, en]
    d_ref, an, bn = oracle.gemm_entries("mxfp8", wq, em, en)
    r = _r(got, d_ref * alpha, an * abs(w["tA"]), bn * abs(w["tB"]))
    _gpu.say(f"  vs the FP4-rate oracle ({len(em)} sampled): max r={r.max():.3e}")
    assert r.max() <= _gpu.tol_bound(K)
    de, ane, bne = oracle.gemm_entries("nvfp4", w, em, en)
    re = _r(got, de, ane, bne)
    _gpu.say(f"  vs the exact NVFP4 oracle: max r={re.max():.3e} mean r={re.mean():.3e}")
    assert re.max() <= 2.0 ** -2 + _gpu.tol_bound(K)


def test_error_bound_on_random_codes():
    """Codes and E4M3 scales over their whole ranges: entry by entry, the
    distance from the exact NVFP4 product stays within the stated bound.  Per
    element the requantisation error is at most e = max(2^-4 |x|, 2^-4 2^E)
    (2^E: the block's E8M0 scale), so a product's error is at most
    |a| e_b + |b| e_a + e_a e_b; the GPU's fp32 sums and bf16 rounding come on
    top."""
    _gpu.say("[nvfp4-fp6] error bound, random codes")
    rng = np.random.default_rng(97)
    M, N, K = 96, 80, 256
    w = _pins.make_w("nvfp4", M, N, K, rng, scale_lo=0x08, scale_hi=0x7E)
    D, ws = run_fp6(w)
    torch.cuda.synchronize()
    de, _, _ = oracle.gemm_full("nvfp4", w, norms=False)
    va, vb = _pins.ref_values("nvfp4", w, "A"), _pins.ref_values("nvfp4", w, "B")
    _, _, sa, sb = _ws_parts(ws, M, N, K)

    def elem_bound(v, e8):
        two_e = np.repeat(np.ldexp(1.0, e8.astype(np.int64) - 127), 32, axis=1)
        return np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -4 * two_e)

    ea, eb = elem_bound(va, sa), elem_bound(vb, sb)
    alpha = abs(w["tA"] * w["tB"])
    bound = alpha * (ea @ np.abs(vb).T + np.abs(va) @ eb.T + ea @ eb.T)
    got = _gpu.d_to_numpy(D)
    gpu_own = 2.0 ** -8 * np.abs(got) + alpha * K * 2.0 ** -22 * ((np.abs(va) + ea) @ (np.abs(vb) + eb).T)
    worst = float(np.max(np.abs(got - de) / (bound + gpu_own)))
    _gpu.say(f"  largest error / bound: {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("M", [300, 2304], ids=["widening", "fp6-rate"])
def test_exact_at_unit_scales(M):
    """Unit E4M3 scales: requantisation is lossless and A times a permutation
    matrix comes out bit for bit equal to the exact NVFP4 product."""
    _gpu.say(f"[nvfp4-fp6] exact at unit scales, M={M}")
    rng = np.random.default_rng(98)
    K = 2304 if M > 300 else 512
    N = K
    a = _pins.random_codes("nvfp4", M, K, rng)
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), rng.permutation(K)] = 0x2
    w = {"fmt": "nvfp4", "M": M, "N": N, "K": K, "A": a["X"], "sA": np.full((M, K // 16), 0x38, np.uint8),
         "B": (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), "sB": np.full((N, K // 16), 0x38, np.uint8),
         "tA": 2.0, "tB": 0.25}
    D, _ = run_fp6(w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(75, M, N, 4096)
    _gpu.check_exact_sampled("nvfp4", w, D, em, en)


def test_requant_every_scale_pair_and_code():
    """One block per row for every pair of finite E4M3 group scales of either
    sign (codes 0x00 .. 0x7E and 0x80 .. 0xFE), each group holding all 16 E2M1
    codes: the E2M3 codes and E8M0 scales bit for bit against the oracle."""
    _gpu.say("[nvfp4-fp6] requantisation over every scale pair")
    s = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    s0, s1 = np.meshgrid(s, s, indexing="ij")
    M, K, N = s0.size, 32, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    rng = np.random.default_rng(99)
    b = _pins.random_codes("nvfp4", N, K, rng)
    w = {"fmt": "nvfp4", "M": M, "N": N, "K": K, "A": np.tile(packed, (M, 1)),
         "sA": np.stack([s0.ravel(), s1.ravel()], axis=1).astype(np.uint8),
         "B": b["X"], "sB": np.full((N, K // 16), 0x38, np.uint8), "tA": 1.0, "tB": 1.0}
    D, ws = run_fp6(w)
    torch.cuda.synchronize()
    a, _, sa, _ = _ws_parts(ws, M, N, K)
    ra, rsa = oracle.requant_nvfp4_e2m3(w["A"], w["sA"], K)
    assert np.array_equal(sa, rsa)
    bad = np.argwhere(a != ra)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:3].tolist()}: {a[tuple(bad[0])]:#x} vs {ra[tuple(bad[0])]:#x}"
