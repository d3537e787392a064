"""GPU grouped GEMMs (mixture-of-experts layout) through the C ABI: every
group's rows of D against the oracle GEMM of that group's operands."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _grouped_w(fmt, sizes, N, K, seed):
    """One A tensor of sum(sizes) rows (one tensor scale for NVFP4) and G
    weight blocks of N rows; group g's tensor scale is tB * 2^-g."""
    G, M = len(sizes), int(sum(sizes))
    w = synth.workload(fmt, M, G * N, K, 100 * seed + 1, 100 * seed + 2)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    w["off"], w["G"], w["Ng"] = off, G, N
    if fmt == "nvfp4":
        w["tBg"] = [w["tB"] * 2.0 ** -g for g in range(G)]
    return w


def _run_grouped(fmt, w):
    d = _gpu.to_dev(w)
    G, N, K = w["G"], w["Ng"], w["K"]
    B = d["B"].reshape(G, N, -1)
    off = w["off"].tolist()
    if fmt == "bf16":
        return dbs.gemm_grouped_bf16(d["A"], B, off)
    sB = d["sB"].reshape(G, N, -1)
    if fmt == "nvfp4":
        return dbs.gemm_grouped_nvfp4(d["A"], d["sA"], w["tA"], B, sB, w["tBg"], off)
    elem = "e4m3" if fmt == "mxfp8" else "e2m1"
    return dbs.gemm_grouped_mx(elem, d["A"], d["sA"], B, sB, off, K=K)


def _group_w(fmt, w, g):
    a, b = int(w["off"][g]), int(w["off"][g + 1])
    N = w["Ng"]
    wg = {"fmt": fmt, "M": b - a, "N": N, "K": w["K"], "A": w["A"][a:b], "B": w["B"][g * N:(g + 1) * N]}
    if fmt != "bf16":
        wg["sA"], wg["sB"] = w["sA"][a:b], w["sB"][g * N:(g + 1) * N]
    if fmt == "nvfp4":
        wg["tA"], wg["tB"] = w["tA"], w["tBg"][g]
    return wg


FMTS = ["bf16", "mxfp8", "mxfp4", "nvfp4"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("sizes,N,K", [
    ([0, 1, 300, 77, 520], 260, 352),      # empty and one-row groups, ragged edges, 256 x 64 tiles
    ([130, 0, 257], 200, 512),             # MX scale rows of whole 16-byte chunks; 4-wave raw NVFP4
    ([200, 0, 700, 64], 5000, 768),        # 395 tiles of 256 x 64: a second persistent round, 3 stages a tile
], ids=["mixed", "aligned", "rounds"])
def test_grouped_matches_oracle(fmt, sizes, N, K):
    _gpu.say(f"[grouped] {fmt} sizes={sizes} N={N} K={K}")
    w = _grouped_w(fmt, sizes, N, K, seed=7)
    D = _run_grouped(fmt, w)
    torch.cuda.synchronize()
    for g in range(w["G"]):
        a, b = int(w["off"][g]), int(w["off"][g + 1])
        if a == b:
            continue
        _gpu.check_full(fmt, _group_w(fmt, w, g), D[a:b])


@pytest.mark.parametrize("fmt", FMTS)
def test_grouped_square_tiles(fmt):
    """Groups large enough for 256 x 256 tiles and more than one persistent
    round; sampled entries of every group."""
    sizes, N, K = [1000, 2500, 0, 1800], 2900, 1024
    _gpu.say(f"[grouped] {fmt} square tiles sizes={sizes}")
    w = _grouped_w(fmt, sizes, N, K, seed=8)
    D = _run_grouped(fmt, w)
    torch.cuda.synchronize()
    for g in range(w["G"]):
        a, b = int(w["off"][g]), int(w["off"][g + 1])
        if a == b:
            continue
        em, en = synth.sample_entries(9 + g, b - a, N, 1024)
        _gpu.check_sampled(fmt, _group_w(fmt, w, g), D[a:b].contiguous(), em, en, label=f"group {g}")


def test_grouped_nvfp4_k_odd_multiple_of_16():
    """NVFP4 groups with K = 80 (an odd multiple of 16)."""
    sizes, N, K = [5, 300, 0, 64], 96, 80
    _gpu.say(f"[grouped] nvfp4 sizes={sizes} N={N} K={K}")
    w = _grouped_w("nvfp4", sizes, N, K, seed=10)
    D = _run_grouped("nvfp4", w)
    torch.cuda.synchronize()
    for g in range(w["G"]):
        a, b = int(w["off"][g]), int(w["off"][g + 1])
        if a < b:
            _gpu.check_full("nvfp4", _group_w("nvfp4", w, g), D[a:b])
