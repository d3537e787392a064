"""GPU quantisers (fp32 -> MXFP8 / MXFP4 / NVFP4 / bf16 codes and scales)
through the C ABI, bit for bit against the oracle's quantisation recipes."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _special_rows(K: int, emax: float) -> np.ndarray:
    """Rows that reach the recipes' corner cases: an all-zero block, signed
    zeros, blocks whose amax is exactly emax * 2^k or just below it, grid
    midpoints (ties) of E4M3 and E2M1 at several scales, values past
    saturation after scaling, and tiny / huge / subnormal fp32 magnitudes."""
    rows = []
    z = np.zeros(K, np.float32)
    rows.append(z.copy())
    r = z.copy(); r[1::2] = -0.0; rows.append(r)
    for k in (-3, 0, 5):
        r = np.full(K, 0.3 * 2.0 ** k, np.float32)
        r[0::32] = emax * 2.0 ** k                                 # amax exactly emax * 2^k
        r[1::32] = np.nextafter(np.float32(emax * 2.0 ** k), np.float32(0))
        rows.append(r)
    # E4M3 and E2M1 grid midpoints (ties), in a block whose amax is the format max
    mids = np.array([1.0625, 1.1875, 0.0029296875, 0.0048828125, 17.0, 240.0, 464.0,
                     0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -1.0625, -0.75, -5.0], np.float32)
    r = np.resize(mids, K).astype(np.float32)
    r[0::32] = emax
    rows.append(r)
    # FP6 grid midpoints: E2M3 (steps 0.125 / 0.25 / 0.5) and E3M2 (0.0625 ... 4)
    mids6 = np.array([1.0625, 1.1875, 4.25, 4.75, 0.0625, 0.1875, 7.25, 7.75, 1.125, 1.375, 0.03125, 0.09375,
                      18.0, 22.0, 26.0, 30.0, -0.1875, -26.0], np.float32)
    r = np.resize(mids6, K).astype(np.float32)
    r[0::32] = emax
    rows.append(r)
    r = np.resize(mids, K).astype(np.float32) * np.float32(2.0 ** -7)
    r[0::32] = emax * 2.0 ** -7
    rows.append(r)
    r = np.linspace(-9.0, 9.0, K).astype(np.float32)              # steps through every binade
    rows.append(r)
    r = np.resize(np.array([1e30, -3e29, 1.0, 1e-30], np.float32), K); rows.append(r)
    r = np.resize(np.array([1e-38, 1e-40, -3e-41, 1.4e-45, 0.0], np.float32), K); rows.append(r)
    return np.stack(rows).astype(np.float32)


def _inputs(K: int, emax: float):
    x = synth.normal(71, 300, K)
    return np.concatenate([x, _special_rows(K, emax)])


@pytest.mark.parametrize("elem,emax", [("e4m3", 448.0), ("e5m2", 57344.0), ("e2m1", 6.0), ("e2m3", 7.5),
                                       ("e3m2", 28.0)])
@pytest.mark.parametrize("K", [32, 1024])
def test_quant_mx_matches_oracle(elem, emax, K):
    _gpu.say(f"[quant] mx {elem} K={K}")
    x = _inputs(K, emax)
    codes, scales = dbs.quant_mx(elem, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.quant_mx(x, elem)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("K", [16, 1024])
@pytest.mark.parametrize("special", [False, True], ids=["normal", "special"])
def test_quant_nvfp4_matches_oracle(K, special):
    _gpu.say(f"[quant] nvfp4 K={K} special={special}")
    x = _inputs(K, 6.0) if special else synth.normal(72, 300, K)
    codes, scales, t = dbs.quant_nvfp4(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    rc, rs, rt = oracle.quant_nvfp4(x)
    assert np.float32(t.item()) == np.float32(rt)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_nvfp4_all_zero():
    _gpu.say("[quant] nvfp4 zero tensor")
    x = np.zeros((8, 64), np.float32)
    codes, scales, t = dbs.quant_nvfp4(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    rc, rs, rt = oracle.quant_nvfp4(x)
    assert t.item() == rt == 1.0
    assert np.array_equal(scales.cpu().numpy(), rs) and np.array_equal(codes.cpu().numpy(), rc)


def test_quant_bf16_matches_oracle():
    _gpu.say("[quant] bf16")
    x = np.concatenate([synth.normal(73, 64, 256), _special_rows(256, 448.0)])
    out = dbs.quant_bf16(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), oracle.quant_bf16(x))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_quantise_then_gemm(fmt):
    """GPU-quantised operands through the GEMM agree with the oracle GEMM on
    the same codes (the two kernels chained on one stream)."""
    _gpu.say(f"[quant] {fmt} quantise then GEMM")
    xa, xb = synth.normal(74, 260, 512), synth.normal(75, 300, 512)
    ta, tb = torch.from_numpy(xa).cuda(), torch.from_numpy(xb).cuda()
    w = {"fmt": fmt, "M": 260, "N": 300, "K": 512}
    if fmt == "nvfp4":
        ca, sa, tA = dbs.quant_nvfp4(ta)
        cb, sb, tB = dbs.quant_nvfp4(tb)
        w.update(tA=float(tA.item()), tB=float(tB.item()))
    else:
        elem = "e4m3" if fmt == "mxfp8" else "e2m1"
        ca, sa = dbs.quant_mx(elem, ta)
        cb, sb = dbs.quant_mx(elem, tb)
    w.update(A=ca.cpu().numpy(), sA=sa.cpu().numpy(), B=cb.cpu().numpy(), sB=sb.cpu().numpy())
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    _gpu.check_full(fmt, w, D)


def test_quantise_e5m2_then_mixed_gemm():
    """GPU-quantised E5M2 A with E4M3 B through gemm_mx_mixed against the
    oracle GEMM on the same codes."""
    _gpu.say("[quant] e5m2 x e4m3 quantise then GEMM")
    xa, xb = synth.normal(76, 260, 512), synth.normal(77, 300, 512)
    ca, sa = dbs.quant_mx("e5m2", torch.from_numpy(xa).cuda())
    cb, sb = dbs.quant_mx("e4m3", torch.from_numpy(xb).cuda())
    D = dbs.gemm_mx_mixed("e5m2", "e4m3", ca, sa, cb, sb, K=512)
    torch.cuda.synchronize()
    w = {"fmt": "mxfp8", "M": 260, "N": 300, "K": 512, "elemA": "e5m2", "elemB": "e4m3",
         "A": ca.cpu().numpy(), "sA": sa.cpu().numpy(), "B": cb.cpu().numpy(), "sB": sb.cpu().numpy()}
    _gpu.check_full("mxfp8", w, D)


def test_quantise_fp6_then_gemm():
    """FP6 codes and scales from the GPU quantiser feed the FP6 GEMM; the
    product matches the oracle on the same codes."""
    _gpu.say("[quant] e2m3 x e3m2 quantise then GEMM")
    xa, xb = synth.normal(81, 260, 512), synth.normal(82, 300, 512)
    ca, sa = dbs.quant_mx("e2m3", torch.from_numpy(xa).cuda())
    cb, sb = dbs.quant_mx("e3m2", torch.from_numpy(xb).cuda())
    D = dbs.gemm_mx_mixed("e2m3", "e3m2", ca, sa, cb, sb, K=512)
    torch.cuda.synchronize()
    w = {"fmt": "mxfp8", "M": 260, "N": 300, "K": 512, "elemA": "e2m3", "elemB": "e3m2",
         "A": ca.cpu().numpy(), "sA": sa.cpu().numpy(), "B": cb.cpu().numpy(), "sB": sb.cpu().numpy()}
    _gpu.check_full("mxfp8", w, D)
