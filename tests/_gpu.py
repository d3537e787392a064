"""Helpers for the GPU parity tests: move encoded operands to the device, call
the HIP path through the C ABI binding, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dense_block_scaled_amd as dbs
import oracle

K_ELEMENT_BITS = {"bf16": 16, "mxfp8": 8, "mxfp4": 4, "nvfp4": 4}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w: dict) -> dict:
    d = {}
    for k in ("A", "B", "sA", "sB"):
        if k in w:
            a = np.ascontiguousarray(w[k])
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            d[k] = t.to("cuda")
    return d


def run(fmt: str, w: dict, dev: dict | None = None, out=None) -> torch.Tensor:
    """Launch the HIP GEMM for workload w; returns the bf16 output tensor."""
    dev = dev or to_dev(w)
    if fmt == "bf16":
        return dbs.gemm_bf16(dev["A"], dev["B"], out=out)
    if fmt == "mxfp8":
        return dbs.gemm_mx("e4m3", dev["A"], dev["sA"], dev["B"], dev["sB"], K=w["K"], out=out)
    if fmt == "mxfp4":
        return dbs.gemm_mx("e2m1", dev["A"], dev["sA"], dev["B"], dev["sB"], K=w["K"], out=out)
    return dbs.gemm_nvfp4(dev["A"], dev["sA"], w["tA"], dev["B"], dev["sB"], w["tB"], out=out)


def d_to_numpy(D: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float64 numpy array (via its bit pattern)."""
    bits = D.view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def d_bits(D: torch.Tensor) -> np.ndarray:
    return D.view(torch.int16).cpu().numpy().view(np.uint16)


def tol_bound(K: int) -> float:
    """Bound on r for a correct fp32-accumulating path with bf16 output:
    bf16 rounding (2^-8 relative to |D| <= ||a|| ||b||) plus K fp32 additions
    (K * 2^-23 relative to sum |a_k b_k| <= ||a|| ||b||)."""
    return 2.0 ** -8 + K * 2.0 ** -23


TOL = 1e-2   # the contract's tolerance on r


def check_full(fmt: str, w: dict, D: torch.Tensor, label: str = "") -> float:
    d_ref, an, bn = oracle.gemm_full(fmt, w)
    r = oracle.rel_errors(d_to_numpy(D), d_ref, an, bn)
    rmax = float(r.max()) if r.size else 0.0
    say(f"  {label} {fmt} M={w['M']} N={w['N']} K={w['K']}: max r={rmax:.3e} mean r={float(r.mean()):.3e}")
    assert np.all(np.isfinite(r)), "non-finite output"
    assert rmax <= TOL, rmax
    assert rmax <= tol_bound(w["K"]), rmax
    return rmax


def check_sampled(fmt: str, w: dict, D: torch.Tensor, em, en, label: str = "") -> float:
    d_ref, an, bn = oracle.gemm_entries(fmt, w, em, en)
    Dn = D.view(torch.int16)
    idx = torch.from_numpy(np.asarray(em) * w["N"] + np.asarray(en)).to(D.device)
    bits = Dn.reshape(-1)[idx].cpu().numpy().view(np.uint16)
    got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = oracle.rel_errors(got, d_ref, an, bn)
    rmax = float(r.max())
    say(f"  {label} {fmt} M={w['M']} N={w['N']} K={w['K']} ({len(em)} sampled): "
        f"max r={rmax:.3e} mean r={float(r.mean()):.3e}")
    assert np.all(np.isfinite(r)), "non-finite output"
    assert rmax <= TOL, rmax
    assert rmax <= tol_bound(w["K"]), rmax
    return rmax


def check_exact(fmt: str, w: dict, D: torch.Tensor) -> None:
    """Every output must equal the bf16 rounding of the oracle's value bit for
    bit (for inputs whose exact result is representable)."""
    d_ref, _, _ = oracle.gemm_full(fmt, w, norms=False)
    want = oracle.encode("bf16", d_ref)
    got = d_bits(D)
    # +0 and -0 are the same value
    same = (got == want) | (((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0))
    bad = np.argwhere(~same)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:5].tolist()}: got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}"


def check_exact_sampled(fmt: str, w: dict, D: torch.Tensor, em, en) -> None:
    """check_exact on the given output entries only (for shapes whose full
    oracle product would take minutes)."""
    d_ref, _, _ = oracle.gemm_entries(fmt, w, em, en)
    want = oracle.encode("bf16", d_ref)
    idx = torch.from_numpy(np.asarray(em) * w["N"] + np.asarray(en)).to(D.device)
    got = D.view(torch.int16).reshape(-1)[idx].cpu().numpy().view(np.uint16)
    same = (got == want) | (((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0))
    bad = np.flatnonzero(~same)
    assert bad.size == 0, (f"{len(bad)} mismatches, first at ({em[bad[0]]}, {en[bad[0]]}): "
                           f"got {got[bad[0]]:#06x} want {want[bad[0]]:#06x}")
