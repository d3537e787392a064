#!/usr/bin/env python3
"""Throughput of the block-scaled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 500] [--fmt bf16]

One step is one GEMM D = bf16((sA.A)(sB.B)^T) of the chosen workload (default:
BF16 at M = N = K = 8192, the metric's shape).  Protocol (after the
benchmarking rules of the "ThunderKittens 2.0" notes, section 5): seeded
N(0,1) inputs encoded once and copied into bit-identical input groups, as many
as needed for the inputs to exceed three times the 256 MB last-level cache;
`warmup` launches cycling the groups; then `steps` back-to-back launches
between two events on the launch stream, with a device synchronisation on
both sides; a 0.5 s pause between workloads.  The same protocol then times
every other workload (reported under "per_format"): BF16 4096^3, MXFP8,
MXFP4 at 8192^3 and 16384^3, NVFP4 square and skinny (256 x 16384 x 8192),
the opt-in lossy FP8- and FP4-rate NVFP4 paths, E4M3 x E2M1 and MXFP6.
With --only, --fmt also names workloads outside that table (the skinny
BF16/MXFP8/MXFP4 shapes, E2M1 x E4M3, E4M3 x E2M1 with K = 8064 on the
widening path, E3M2 x E4M3 widened, BF16 on the decoupled-ring kernel
with A released early or at the stage's end), and
--layout hands A and/or B over
MN-major.

Each line is priced against the dense MFMA peak of the arithmetic its
kernels run (NVFP4's exact path multiplies in fp16, and is also quoted
against the FP4 peak the format would have on hardware taking its scales),
carries the GPU clock read while the kernel runs, and the oracle's largest
relative error r on 4096 seeded output entries of the timed result.

Printed: one JSON line with the throughput (TFLOP/s), the roofline fraction
of the timed kernel, and the CPU oracle timed on a bounded sample of the same
workload (rows 0..R-1, every column), which doubles as a parity check of the
timed output.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

LLC_BYTES = 256 * 2 ** 20                      # MI355X Infinity Cache (MALL)
HBM_GBS = 8000.0
CLOCK_PEAK_MHZ = 2400.0                        # the clock the datasheet peaks assume
# MI355X dense MFMA peaks (TFLOP/s), by the arithmetic the MFMAs run
PEAK = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0, "fp6": 10100.0, "fp4": 10100.0}
ELEM_BITS = {"bf16": 16, "mxfp8": 8, "mxfp4": 4, "nvfp4": 4}
BLOCK = {"bf16": 0, "mxfp8": 32, "mxfp4": 32, "nvfp4": 16}

# workload -> config index (seeds 100c+1, 100c+2 for A, B; 100c+3 for the
# sampled entries), shape, input encoding, entry point, MFMA arithmetic,
# MX element formats of A and B where they differ from the encoding's own
W = {
    "bf16": dict(c=1, shape=(8192, 8192, 8192), enc="bf16", kernel="bf16", mfma="bf16"),
    "bf16_4096": dict(c=1, shape=(4096, 4096, 4096), enc="bf16", kernel="bf16", mfma="bf16"),
    "mxfp8": dict(c=2, shape=(8192, 8192, 8192), enc="mxfp8", kernel="mxfp8", mfma="fp8"),
    "mxfp4": dict(c=3, shape=(8192, 8192, 8192), enc="mxfp4", kernel="mxfp4", mfma="fp4"),
    "mxfp4_16384": dict(c=3, shape=(16384, 16384, 16384), enc="mxfp4", kernel="mxfp4", mfma="fp4"),
    "nvfp4": dict(c=4, shape=(8192, 8192, 8192), enc="nvfp4", kernel="nvfp4", mfma="fp16", alt="fp4"),
    "nvfp4_skinny": dict(c=4, shape=(256, 16384, 8192), enc="nvfp4", kernel="nvfp4", mfma="fp16", alt="fp4"),
    "nvfp4_fp8": dict(c=4, shape=(8192, 8192, 8192), enc="nvfp4", kernel="nvfp4_fp8", mfma="fp8", alt="fp4"),
    "nvfp4_fp8_skinny": dict(c=4, shape=(256, 16384, 8192), enc="nvfp4", kernel="nvfp4_fp8", mfma="fp8",
                             alt="fp4"),
    "nvfp4_fp6": dict(c=4, shape=(8192, 8192, 8192), enc="nvfp4", kernel="nvfp4_fp6", mfma="fp6", alt="fp4"),
    "nvfp4_fp6_skinny": dict(c=4, shape=(256, 16384, 8192), enc="nvfp4", kernel="nvfp4_fp6", mfma="fp6",
                             alt="fp4"),
    "mx_e4m3_e2m1": dict(c=2, shape=(8192, 8192, 8192), enc="mxfp8", kernel="mx_mixed", mfma="fp8",
                         elems=("e4m3", "e2m1")),
    "mx_e2m3_e2m3": dict(c=2, shape=(8192, 8192, 8192), enc="mxfp8", kernel="mx_mixed", mfma="fp6",
                         elems=("e2m3", "e2m3")),
}
# timed only when named with --fmt (not in the default table): the other
# tilings and element pairings the library routes to
W.update({
    "bf16_skinny": dict(c=1, shape=(256, 16384, 8192), enc="bf16", kernel="bf16", mfma="bf16"),
    "mxfp8_skinny": dict(c=2, shape=(256, 16384, 8192), enc="mxfp8", kernel="mxfp8", mfma="fp8"),
    "mxfp4_skinny": dict(c=3, shape=(256, 16384, 8192), enc="mxfp4", kernel="mxfp4", mfma="fp4"),
    "mx_e2m1_e4m3": dict(c=2, shape=(8192, 8192, 8192), enc="mxfp8", kernel="mx_mixed", mfma="fp8",
                         elems=("e2m1", "e4m3")),
    "mx_e4m3_e2m1_skinny": dict(c=2, shape=(256, 16384, 8192), enc="mxfp8", kernel="mx_mixed", mfma="fp8",
                                elems=("e4m3", "e2m1")),
    "mx_e4m3_e2m1_k8064": dict(c=2, shape=(8192, 8192, 8064), enc="mxfp8", kernel="mx_mixed", mfma="fp8",
                               elems=("e4m3", "e2m1")),
    "mx_e3m2_e4m3": dict(c=2, shape=(8192, 8192, 8192), enc="mxfp8", kernel="mx_mixed", mfma="fp8",
                         elems=("e3m2", "e4m3")),
    "bf16_rings_early_a": dict(c=1, shape=(8192, 8192, 8192), enc="bf16", kernel="bf16_ea", mfma="bf16"),
    "bf16_rings_late_a": dict(c=1, shape=(8192, 8192, 8192), enc="bf16", kernel="bf16_el", mfma="bf16"),
    "bf16_rings_early_a_4096": dict(c=1, shape=(4096, 4096, 4096), enc="bf16", kernel="bf16_ea", mfma="bf16"),
    "bf16_rings_late_a_4096": dict(c=1, shape=(4096, 4096, 4096), enc="bf16", kernel="bf16_el", mfma="bf16"),
    "bf16_16384": dict(c=1, shape=(16384, 16384, 16384), enc="bf16", kernel="bf16", mfma="bf16"),
    "bf16_rings_early_a_16384": dict(c=1, shape=(16384, 16384, 16384), enc="bf16", kernel="bf16_ea", mfma="bf16"),
    "bf16_rings_late_a_16384": dict(c=1, shape=(16384, 16384, 16384), enc="bf16", kernel="bf16_el", mfma="bf16"),
})
ORDER = ["bf16", "bf16_4096", "mxfp8", "mxfp4", "mxfp4_16384", "nvfp4", "nvfp4_skinny", "nvfp4_fp8",
         "nvfp4_fp8_skinny", "nvfp4_fp6", "nvfp4_fp6_skinny", "mx_e4m3_e2m1", "mx_e2m3_e2m3"]
PEAK_NOTE = {
    "nvfp4": "exact NVFP4 runs its products on fp16 MFMA (no FP8/FP4 operand holds an E2M1 x E4M3 product): "
             "frac_mfma_peak is against the fp16 dense peak; frac_fp4_peak against the FP4 dense peak",
    "nvfp4_skinny": "as nvfp4; frac_path_roofline is against min(HBM time, fp16 MFMA time) of this shape",
    "nvfp4_fp8": "opt-in lossy FP8-rate NVFP4 (gemm_nvfp4_fp8): requantisation to MXFP8 plus the MXFP8 GEMM, "
                 "both inside the timed launch; priced at the fp8 dense peak; max_r is against the oracle of "
                 "the same method, max_r_vs_exact against the exact NVFP4 oracle",
    "nvfp4_fp6": "opt-in lossy FP4-rate NVFP4 (gemm_nvfp4_fp6): requantisation to MXFP6 E2M3 plus the FP6 GEMM "
                 "(the FP6-rate kernel on 256 x 256 tiles), both inside the timed launch; priced at the FP6 dense "
                 "peak (= FP4); max_r is against the oracle of the same method, max_r_vs_exact against the exact "
                 "NVFP4 oracle",
    "nvfp4_fp6_skinny": "as nvfp4_fp6; this shape's 64 square tiles are too few for the FP6-rate kernel, so its "
                        "GEMM runs widened to 8 bits on 256 x 64 tiles",
    "mx_e4m3_e2m1": "E4M3 A x E2M1 B (gemm_mx_mixed, packed E2M1 on the MFMA's mixed formats): priced at the "
                    "fp8 dense peak, the rate its MFMAs run at",
    "mx_e2m3_e2m3": "MXFP6 (E2M3 both sides): priced at the FP6 dense peak",
}
KERNEL_SOURCES = ["dense_block_scaled_amd/csrc/" + f for f in
                  ("gemm_kernel.h", "launch.h", "gemm.hip", "gemm_bf16.hip", "gemm_mxfp8.hip", "gemm_mx8_e5m2.hip",
                   "gemm_mx8_fp4.hip", "gemm_mxfp4.hip", "gemm_nvfp4.hip", "gemm_mxfp6.hip", "quant.hip",
                   "gemm_bf16_ea.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(name, M, N, K):
    """A + B + scales + D, each moved once, for workload `name`."""
    spec = W[name]
    enc = spec["enc"]
    ea, eb = spec.get("elems", (None, None))
    sub_bits = {"e2m1": 4, "e2m3": 6, "e3m2": 6, "e4m3": 8}
    bits_a = sub_bits.get(ea, ELEM_BITS[enc])
    bits_b = sub_bits.get(eb, ELEM_BITS[enc])
    b = (M * bits_a + N * bits_b) * K // 8 + M * N * 2
    if BLOCK[enc]:
        b += (M + N) * (K // BLOCK[enc])
    return b


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update((ROOT / p).read_bytes())
    return h.hexdigest()[:16]


def git_sha():
    """HEAD's commit id, read from the repository's .git files (None where the
    tree carries no git metadata, as in a copied snapshot)."""
    g = ROOT / ".git"
    try:
        head = (g / "HEAD").read_text().strip()
        if not head.startswith("ref: "):
            return head or None
        ref = head[5:]
        if (g / ref).exists():
            return (g / ref).read_text().strip() or None
        for line in (g / "packed-refs").read_text().splitlines():
            if line.endswith(" " + ref):
                return line.split()[0]
    except OSError:
        return None
    return None


def provenance(name):
    """Where a record's numbers come from: the seeds of the workload's inputs
    (A and its scales, B and its scales) and of its sampled output entries,
    the hash of the kernel sources, the commit."""
    c = W[name]["c"]
    return {"seeds": {"A": 100 * c + 1, "B": 100 * c + 2, "sampled_entries": 100 * c + 3},
            "kernel_source_sha": kernel_source_hash(), "git_sha": git_sha()}


def traffic_for(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except ValueError:
        return None
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    e = d.get("workloads", {}).get(workload)
    return None if e is None else e.get("hbm_bytes_per_launch")


def make_inputs(name):
    import synth
    spec = W[name]
    M, N, K = spec["shape"]
    c = spec["c"]
    return synth.workload(spec["enc"], M, N, K, 100 * c + 1, 100 * c + 2, *spec.get("elems", ()))


def to_mn(enc, X):
    """K-major operand storage (rows, K) -> MN-major storage (K, rows); E2M1
    codes are re-packed two per byte along the rows."""
    if enc in ("bf16", "mxfp8"):
        return np.ascontiguousarray(X.T)
    codes = np.empty((X.shape[0], 2 * X.shape[1]), np.uint8)
    codes[:, 0::2] = X & 0xF
    codes[:, 1::2] = X >> 4
    t = np.ascontiguousarray(codes.T)
    return (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)


def to_device(w, lay="kk"):
    import torch
    out = {}
    for k in ("A", "B", "sA", "sB"):
        if k in w:
            a = np.ascontiguousarray(w[k])
            if (k == "A" and lay[0] == "m") or (k == "B" and lay[1] == "m"):
                a = to_mn(w["fmt"], a)
            out[k] = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
    return out


def launcher(name, w, dev, out, lay="kk"):
    import dense_block_scaled_amd as dbs
    K = w["K"]
    kern = W[name]["kernel"]
    la, lb = int(lay[0] == "m"), int(lay[1] == "m")
    if kern == "bf16":
        return lambda: dbs.gemm_bf16(dev["A"], dev["B"], out=out, la=la, lb=lb)
    if kern in ("bf16_ea", "bf16_el"):
        early = kern == "bf16_ea"
        return lambda: dbs.gemm_bf16_decoupled(dev["A"], dev["B"], out=out, early_release_a=early)
    if kern == "mxfp8":
        return lambda: dbs.gemm_mx("e4m3", dev["A"], dev["sA"], dev["B"], dev["sB"], K=K, out=out, la=la, lb=lb)
    if kern == "mxfp4":
        return lambda: dbs.gemm_mx("e2m1", dev["A"], dev["sA"], dev["B"], dev["sB"], K=K, out=out, la=la, lb=lb)
    if kern == "mx_mixed":
        ea, eb = W[name]["elems"]
        return lambda: dbs.gemm_mx_mixed(ea, eb, dev["A"], dev["sA"], dev["B"], dev["sB"], K=K, out=out)
    tA, tB = w["tA"], w["tB"]
    if kern == "nvfp4_fp8":
        import torch
        ws = torch.empty(dbs.nvfp4_fp8_workspace_bytes(w["M"], w["N"], K), dtype=torch.uint8, device="cuda")
        return lambda: dbs.gemm_nvfp4_fp8(dev["A"], dev["sA"], tA, dev["B"], dev["sB"], tB, out=out, workspace=ws)
    if kern == "nvfp4_fp6":
        import torch
        ws = torch.empty(dbs.nvfp4_fp6_workspace_bytes(w["M"], w["N"], K), dtype=torch.uint8, device="cuda")
        return lambda: dbs.gemm_nvfp4_fp6(dev["A"], dev["sA"], tA, dev["B"], dev["sB"], tB, out=out, workspace=ws)
    return lambda: dbs.gemm_nvfp4(dev["A"], dev["sA"], tA, dev["B"], dev["sB"], tB, out=out, la=la, lb=lb)


class ClockReader:
    """The GPU's current graphics clock (MHz) through amdsmi; None where the
    management library cannot be used."""

    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            self.amdsmi, self.h = amdsmi, (hs[0] if hs else None)
        except Exception as e:  # no management library access: no clock in the record
            log(f"[bench] no GPU clock readings: {e}")

    def read(self):
        """(mean of the per-XCD current graphics clocks in MHz, GFX activity
        in %) from the SMU's metrics table, or None."""
        if self.h is None:
            return None
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        except Exception:
            return None
        act = m.get("average_gfx_activity")
        act = float(act) if isinstance(act, (int, float)) else None
        xcd = m.get("current_gfxclks")
        if isinstance(xcd, (list, tuple)):
            v = [float(x) for x in xcd if isinstance(x, (int, float)) and 0 < x < 10000]
            if v:
                return sum(v) / len(v), act
        x = m.get("current_gfxclk")
        if isinstance(x, (int, float)) and 0 < x < 10000:
            return float(x), act
        return None


def clock_under_load(clock, call, seconds=1.6):
    """Median graphics clock while `call` runs back to back for ~seconds (a
    window of its own after the timed one).  The metrics table refreshes
    about once a second, so only readings taken while it reports the GPU
    busy (activity >= 80%) count; None if there are none."""
    import torch
    if clock is None or clock.h is None:
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            r = clock.read()
            if r and r[1] is not None and r[1] >= 80:
                samples.append(r[0])
            time.sleep(0.005)

    th = threading.Thread(target=poll)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(4):
            call()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    return float(np.median(samples)) if samples else None


def time_gemm(name, w, steps, warmup, clock=None, lay="kk"):
    """Protocol timing; returns (avg seconds per launch, groups, output tensor,
    clock MHz under load)."""
    import torch
    M, N, K = w["M"], w["N"], w["K"]
    in_bytes = algorithmic_bytes(name, M, N, K) - M * N * 2
    groups = 1 if in_bytes >= 3 * LLC_BYTES else (3 * LLC_BYTES) // in_bytes + 1
    dev0 = to_device(w, lay)
    devs = [dev0] + [{k: v.clone() for k, v in dev0.items()} for _ in range(groups - 1)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    calls = [launcher(name, w, d, out, lay) for d in devs]
    torch.cuda.synchronize()
    for i in range(warmup):
        calls[i % groups]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        calls[i % groups]()
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / 1e3 / steps
    mhz = clock_under_load(clock, lambda: [c() for c in calls])
    # leave the group-0 result in `out` for the parity checks
    calls[0]()
    torch.cuda.synchronize()
    return avg, groups, out, mhz


def gather(D, em, en, N):
    import torch
    idx = torch.from_numpy(np.asarray(em) * N + np.asarray(en)).to(D.device)
    bits = D.view(torch.int16).reshape(-1)[idx].cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def parity_sample(name, w, D):
    """Largest r of the timed output against the oracle on 4096 seeded
    entries (the structured rows/columns and uniform draws).  The FP8-rate
    path is compared with the oracle of its own method, and its error against
    the exact NVFP4 product is returned beside it."""
    import oracle
    import synth
    spec = W[name]
    M, N, K = w["M"], w["N"], w["K"]
    em, en = synth.sample_entries(100 * spec["c"] + 3, M, N)
    got = gather(D, em, en, N)
    d, an, bn = oracle.gemm_entries(spec["enc"], w, em, en)
    r_exact = float(np.max(oracle.rel_errors(got, d, an, bn)))
    if spec["kernel"] not in ("nvfp4_fp8", "nvfp4_fp6"):
        return r_exact, None
    wq = oracle.nvfp4_fp8_workload(w) if spec["kernel"] == "nvfp4_fp8" else oracle.nvfp4_fp6_workload(w)
    dq, aq, bq = oracle.gemm_entries("mxfp8", wq, em, en)
    alpha = float(w["tA"]) * float(w["tB"])
    r = float(np.max(oracle.rel_errors(got, dq * alpha, aq * abs(alpha), bq)))
    return r, r_exact


def cpu_baseline(name, w, D, target_s=12.0):
    """The oracle timed on rows 0..R-1 (every column) of the same workload,
    R sized for ~target_s of CPU work; also checks those GPU outputs."""
    import torch
    import oracle
    M, N, K = w["M"], w["N"], w["K"]
    enc = W[name]["enc"]
    threads = oracle.default_threads()

    def entries(r0, r1):
        em = np.repeat(np.arange(r0, r1, dtype=np.int64), N)
        en = np.tile(np.arange(N, dtype=np.int64), r1 - r0)
        return em, en

    em, en = entries(0, 2)
    t = time.perf_counter()
    oracle.gemm_entries(enc, w, em, en, nthreads=threads)
    per_row = max((time.perf_counter() - t) / 2, 1e-4)
    R = int(min(max(target_s / per_row, 4), M))
    em, en = entries(0, R)
    t = time.perf_counter()
    d_ref, an, bn = oracle.gemm_entries(enc, w, em, en, nthreads=threads)
    dt = time.perf_counter() - t
    bits = D[:R].reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)
    got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = oracle.rel_errors(got, d_ref, an, bn)
    flops = 2.0 * em.size * K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{R - 1} x all {N} columns ({em.size} entries, K={K}) of the {enc} "
                  f"{M}x{N}x{K} GEMM; fp64 C oracle, {dt:.1f} s wall",
        "seconds": dt,
    }, float(np.max(r))


def measure(name, steps, warmup, clock, lay="kk"):
    t = time.perf_counter()
    w = make_inputs(name)
    M, N, K = w["M"], w["N"], w["K"]
    log(f"[bench] {name} {M}x{N}x{K}: inputs ready in {time.perf_counter() - t:.1f} s")
    avg, groups, D, mhz = time_gemm(name, w, steps, warmup, clock, lay)
    tflops = 2.0 * M * N * K / avg / 1e12
    gbs = algorithmic_bytes(name, M, N, K) / avg / 1e9
    log(f"[bench] {name}: {avg * 1e6:.1f} us/launch, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s, {groups} input groups, "
        f"clock {mhz if mhz else 'n/a'} MHz")
    return w, D, avg, groups, tflops, gbs, mhz


def record(name, w, avg, tflops, gbs, mhz, r, r_exact):
    spec = W[name]
    M, N, K = w["M"], w["N"], w["K"]
    peak = PEAK[spec["mfma"]]
    e = {"workload": f"{name}_gemm_{M}x{N}x{K}", "us": round(avg * 1e6, 2), "tflops": round(tflops, 2),
         "mfma_dtype": spec["mfma"], "peak_tflops": peak, "frac_mfma_peak": round(tflops / peak, 4),
         "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_GBS, 4),
         "sclk_mhz": round(mhz, 0) if mhz else None,
         "frac_mfma_peak_at_sclk": round(tflops / (peak * mhz / CLOCK_PEAK_MHZ), 4) if mhz else None,
         "max_r": r, "seeds": provenance(name)["seeds"]}
    if "alt" in spec:
        e["frac_" + spec["alt"] + "_peak"] = round(tflops / PEAK[spec["alt"]], 4)
    if name.endswith("skinny"):
        t_min = max(algorithmic_bytes(name, M, N, K) / (HBM_GBS * 1e9), 2.0 * M * N * K / (peak * 1e12))
        e["frac_path_roofline"] = round(t_min / avg, 4)
    if r_exact is not None:
        e["max_r_vs_exact"] = r_exact
    return e


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--fmt", default="bf16", choices=list(W),
                    help="workload to time (nvfp4_skinny: the 256x16384x8192 NVFP4 GEMM)")
    ap.add_argument("--only", action="store_true", help="time only --fmt (no per_format table)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-clock", action="store_true", help="skip the GPU-clock window (for profiled runs)")
    ap.add_argument("--layout", default="kk", choices=["kk", "mk", "km", "mm"],
                    help="operand storage of A and B: k K-major (rows x K), m MN-major (K x rows); "
                         "BF16, MXFP8, MXFP4 and NVFP4 workloads, with --only")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run 5 device copies of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import dense_block_scaled_amd as dbs
    dbs.lib()
    clock = None if args.no_clock else ClockReader()

    fmt = args.fmt
    lay = args.layout
    if lay != "kk" and (not args.only or W[fmt]["kernel"] not in ("bf16", "mxfp8", "mxfp4", "nvfp4")):
        print("--layout takes a BF16, MXFP8, MXFP4 or NVFP4 workload and --only", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w, D, avg, groups, tflops, gbs, mhz = measure(fmt, args.steps, args.warmup, clock, lay)
    r, r_exact = parity_sample(fmt, w, D)
    head = record(fmt, w, avg, tflops, gbs, mhz, r, r_exact)
    M, N, K = w["M"], w["N"], w["K"]
    workload = f"{fmt}_gemm_{M}x{N}x{K}" + ("" if lay == "kk" else "_" + lay)
    storage = {"kk": "A MxK, B NxK (K-major)", "mk": "A KxM (MN-major), B NxK", "km": "A MxK, B KxN (MN-major)",
               "mm": "A KxM, B KxN (both MN-major)"}[lay]
    peak = PEAK[W[fmt]["mfma"]]
    result = {
        "metric": "TFLOP/s per GEMM (BF16/MXFP8/MXFP4) at 8192^3 and % of dtype MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W[fmt]["enc"],
        "data": "synthetic: seeded N(0,1) (PCG64), encoded per the format's recipe",
        "config": {"workload": workload, "format": fmt, "M": M, "N": N, "K": K,
                   "layout": storage + ", D MxN bf16", "input_groups": groups},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic_for(workload)},
        "sclk_mhz": head["sclk_mhz"],
        "parity_sample_max_r": r,
        "provenance": provenance(fmt),
    }
    if not args.no_cpu:
        cb, rmax = cpu_baseline(fmt, w, D)
        result["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v)
                                  for k, v in cb.items() if k != "seconds"}
        result["parity_rows_max_r"] = rmax
        log(f"[bench] cpu baseline {cb['value'] * 1e3:.3f} GFLOP/s on {cb['cores']} threads; "
            f"rows max r {rmax:.2e}")
    del D
    if not args.only:
        per = [] if fmt in ORDER else [head]
        for f in ORDER:
            if f == fmt:
                per.append(head)
                continue
            time.sleep(0.5)
            wf, Df, af, _, tf, gf, mf = measure(f, args.steps, args.warmup, clock)
            rf, rfe = parity_sample(f, wf, Df)
            log(f"[bench] {f}: sampled max r {rf:.2e}" + (f" (vs exact {rfe:.2e})" if rfe is not None else ""))
            per.append(record(f, wf, af, tf, gf, mf, rf, rfe))
            del Df, wf
            torch.cuda.empty_cache()
        result["per_format"] = per
        result["peak_notes"] = PEAK_NOTE
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
