#!/usr/bin/env python3
"""Throughput of the block-scaled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 500] [--fmt bf16]

One step is one GEMM D = bf16((sA.A)(sB.B)^T) of the chosen format at
M = N = K = 8192 (default: BF16).  Protocol (after the benchmarking rules of
the "ThunderKittens 2.0" notes, section 5): seeded N(0,1) inputs encoded once
and copied into bit-identical input groups, as many as needed for the inputs
to exceed three times the 256 MB last-level cache; `warmup` launches cycling
the groups; then `steps` back-to-back launches between two events on the
launch stream, with a device synchronisation on both sides; a 0.5 s pause
between kernels.  The same protocol then times the other formats at their
shapes (reported under "per_format"), among them the opt-in lossy FP8-rate
NVFP4 path (nvfp4_fp8: requantisation and MXFP8 GEMM in each timed launch).

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
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

LLC_BYTES = 256 * 2 ** 20                      # MI355X Infinity Cache (MALL)
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "nvfp4": 2500.0, "nvfp4_fp8": 5000.0,
               "mx_e4m3_e2m1": 5000.0, "mx_e2m3_e2m3": 5000.0}
PEAK_NOTE = {"nvfp4": "exact NVFP4 runs on fp16 MFMA: priced at the bf16/fp16 dense peak",
             "nvfp4_fp8": "opt-in lossy FP8-rate NVFP4 (gemm_nvfp4_fp8): requantisation to MXFP8 plus the MXFP8 "
                          "GEMM, both inside the timed launch; priced at the fp8 dense peak",
             "mx_e4m3_e2m1": "E4M3 A x E2M1 B (gemm_mx_mixed, packed E2M1 on the MFMA's mixed formats): "
                             "priced at the fp8 dense peak, the rate its MFMAs run at",
             "mx_e2m3_e2m3": "MXFP6 (E2M3 both sides, gemm_mx): widened to E4M3 on the way into LDS and "
                             "multiplied at the fp8 rate; priced at the fp8 dense peak"}
HBM_GBS = 8000.0
ELEM_BITS = {"bf16": 16, "mxfp8": 8, "mxfp4": 4, "nvfp4": 4}
BLOCK = {"bf16": 0, "mxfp8": 32, "mxfp4": 32, "nvfp4": 16}
# config index -> seeds 100c+1, 100c+2 (A, B); sampling seed 100c+3
CONFIGS = {
    "bf16": (1, 8192, 8192, 8192),
    "bf16_4096": (1, 4096, 4096, 4096),
    "mxfp8": (2, 8192, 8192, 8192),
    "mxfp4": (3, 8192, 8192, 8192),
    "nvfp4": (4, 8192, 8192, 8192),
    "nvfp4_skinny": (4, 256, 16384, 8192),
    "nvfp4_fp8": (4, 8192, 8192, 8192),
    "nvfp4_fp8_skinny": (4, 256, 16384, 8192),
    "mx_e4m3_e2m1": (2, 8192, 8192, 8192),
    "mx_e2m3_e2m3": (2, 8192, 8192, 8192),
}
# MX element formats of A and B where they differ from the format's own
MX_ELEMS = {"mx_e4m3_e2m1": ("e4m3", "e2m1"), "mx_e2m3_e2m3": ("e2m3", "e2m3")}
# the encoding each workload's inputs take, and the entry point it times
INPUT_FMT = {"bf16_4096": "bf16", "nvfp4_skinny": "nvfp4", "nvfp4_fp8": "nvfp4", "nvfp4_fp8_skinny": "nvfp4", "mx_e4m3_e2m1": "mxfp8",
             "mx_e2m3_e2m3": "mxfp8"}
KERNEL_OF = {"bf16_4096": "bf16", "nvfp4_skinny": "nvfp4", "nvfp4_fp8_skinny": "nvfp4_fp8"}


def input_fmt(fmt):
    return INPUT_FMT.get(fmt, fmt)


def kernel_of(fmt):
    return KERNEL_OF.get(fmt, fmt)
KERNEL_SOURCES = ["dense_block_scaled_amd/csrc/" + f for f in
                  ("gemm_kernel.h", "launch.h", "gemm.hip", "gemm_bf16.hip", "gemm_mxfp8.hip", "gemm_mx8_e5m2.hip",
                   "gemm_mx8_fp4.hip", "gemm_mxfp4.hip", "gemm_nvfp4.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(fmt, M, N, K):
    """A + B + scales + D, each moved once, for workload (or format) fmt."""
    base = input_fmt(fmt)
    ea, eb = MX_ELEMS.get(fmt, (None, None))
    sub_bits = {"e2m1": 4, "e2m3": 6, "e3m2": 6}
    bits_a = sub_bits.get(ea, ELEM_BITS[base])
    bits_b = sub_bits.get(eb, ELEM_BITS[base])
    b = (M * bits_a + N * bits_b) * K // 8 + M * N * 2
    if BLOCK[base]:
        b += (M + N) * (K // BLOCK[base])
    return b


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update((ROOT / p).read_bytes())
    return h.hexdigest()[:16]


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


def make_inputs(fmt, cfg):
    import synth
    c, M, N, K = cfg
    w = synth.workload(input_fmt(fmt), M, N, K, 100 * c + 1, 100 * c + 2, *MX_ELEMS.get(fmt, ()))
    return w


def to_device(w):
    import torch
    out = {}
    for k in ("A", "B", "sA", "sB"):
        if k in w:
            a = np.ascontiguousarray(w[k])
            out[k] = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
    return out


def launcher(fmt, w, dev, out):
    import dense_block_scaled_amd as dbs
    K = w["K"]
    if fmt == "bf16":
        return lambda: dbs.gemm_bf16(dev["A"], dev["B"], out=out)
    if fmt == "mxfp8":
        return lambda: dbs.gemm_mx("e4m3", dev["A"], dev["sA"], dev["B"], dev["sB"], K=K, out=out)
    if fmt == "mxfp4":
        return lambda: dbs.gemm_mx("e2m1", dev["A"], dev["sA"], dev["B"], dev["sB"], K=K, out=out)
    if fmt in MX_ELEMS:
        ea, eb = MX_ELEMS[fmt]
        return lambda: dbs.gemm_mx_mixed(ea, eb, dev["A"], dev["sA"], dev["B"], dev["sB"], K=K, out=out)
    tA, tB = w["tA"], w["tB"]
    if fmt == "nvfp4_fp8":
        import torch
        ws = torch.empty(dbs.nvfp4_fp8_workspace_bytes(w["M"], w["N"], K), dtype=torch.uint8, device="cuda")
        return lambda: dbs.gemm_nvfp4_fp8(dev["A"], dev["sA"], tA, dev["B"], dev["sB"], tB, out=out, workspace=ws)
    return lambda: dbs.gemm_nvfp4(dev["A"], dev["sA"], tA, dev["B"], dev["sB"], tB, out=out)


def time_gemm(fmt, w, steps, warmup):
    """Protocol timing; returns (avg seconds per launch, groups, output tensor)."""
    import torch
    M, N, K = w["M"], w["N"], w["K"]
    in_bytes = algorithmic_bytes(fmt, M, N, K) - M * N * 2
    groups = 1 if in_bytes >= 3 * LLC_BYTES else (3 * LLC_BYTES) // in_bytes + 1
    dev0 = to_device(w)
    devs = [dev0] + [{k: v.clone() for k, v in dev0.items()} for _ in range(groups - 1)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    calls = [launcher(kernel_of(fmt), w, d, out) for d in devs]
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
    # leave the group-0 result in `out` for the parity sample
    calls[0]()
    torch.cuda.synchronize()
    return avg, groups, out


def cpu_baseline(fmt, w, D, target_s=12.0):
    """The oracle timed on rows 0..R-1 (every column) of the same workload,
    R sized for ~target_s of CPU work; also checks those GPU outputs."""
    import torch
    import oracle
    M, N, K = w["M"], w["N"], w["K"]
    base = input_fmt(fmt)
    threads = oracle.default_threads()

    def entries(r0, r1):
        em = np.repeat(np.arange(r0, r1, dtype=np.int64), N)
        en = np.tile(np.arange(N, dtype=np.int64), r1 - r0)
        return em, en

    em, en = entries(0, 2)
    t = time.perf_counter()
    oracle.gemm_entries(base, w, em, en, nthreads=threads)
    per_row = max((time.perf_counter() - t) / 2, 1e-4)
    R = int(min(max(target_s / per_row, 4), M))
    em, en = entries(0, R)
    t = time.perf_counter()
    d_ref, an, bn = oracle.gemm_entries(base, w, em, en, nthreads=threads)
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
        "sample": f"rows 0..{R - 1} x all {N} columns ({em.size} entries, K={K}) of the {base} "
                  f"{M}x{N}x{K} GEMM; fp64 C oracle, {dt:.1f} s wall",
        "seconds": dt,
    }, float(np.max(r))


def measure(fmt, steps, warmup):
    cfg = CONFIGS[fmt]
    t = time.perf_counter()
    w = make_inputs(fmt, cfg)
    log(f"[bench] {fmt} {cfg[1]}x{cfg[2]}x{cfg[3]}: inputs ready in {time.perf_counter() - t:.1f} s")
    avg, groups, D = time_gemm(fmt, w, steps, warmup)
    M, N, K = w["M"], w["N"], w["K"]
    tflops = 2.0 * M * N * K / avg / 1e12
    gbs = algorithmic_bytes(fmt, M, N, K) / avg / 1e9
    log(f"[bench] {fmt}: {avg * 1e6:.1f} us/launch, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s, {groups} input groups")
    return w, D, avg, groups, tflops, gbs


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--fmt", default="bf16", choices=list(CONFIGS),
                    help="workload to time (nvfp4_skinny: the 256x16384x8192 NVFP4 GEMM)")
    ap.add_argument("--only", action="store_true", help="time only --fmt (no per_format table)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run 5 device copies of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import dense_block_scaled_amd as dbs
    dbs.lib()

    fmt = args.fmt
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w, D, avg, groups, tflops, gbs = measure(fmt, args.steps, args.warmup)
    M, N, K = w["M"], w["N"], w["K"]
    workload = f"{fmt}_gemm_{M}x{N}x{K}"
    peak = PEAK_TFLOPS[kernel_of(fmt)]
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
        "dtype": input_fmt(fmt),
        "data": "synthetic: seeded N(0,1) (PCG64), encoded per the format's recipe",
        "config": {"workload": workload, "format": fmt, "M": M, "N": N, "K": K,
                   "layout": "A MxK, B NxK (K-major), D MxN bf16", "input_groups": groups},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic_for(workload)},
    }
    if not args.no_cpu:
        cb, rmax = cpu_baseline(fmt, w, D)
        result["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v)
                                  for k, v in cb.items() if k != "seconds"}
        result["parity_sample_max_r"] = rmax
        log(f"[bench] cpu baseline {cb['value'] * 1e3:.3f} GFLOP/s on {cb['cores']} threads; "
            f"sample max r {rmax:.2e}")
    if not args.only:
        per = []
        for f in ["bf16", "bf16_4096", "mxfp8", "mxfp4", "nvfp4", "nvfp4_skinny", "nvfp4_fp8", "nvfp4_fp8_skinny",
                  "mx_e4m3_e2m1", "mx_e2m3_e2m3"]:
            if f == fmt:
                entry_t, entry_gbs, entry_avg = tflops, gbs, avg
                wf = w
            else:
                time.sleep(0.5)
                wf, _, entry_avg, _, entry_t, entry_gbs = measure(f, args.steps, args.warmup)
            per.append({"workload": f"{f}_gemm_{wf['M']}x{wf['N']}x{wf['K']}",
                        "us": round(entry_avg * 1e6, 2), "tflops": round(entry_t, 2),
                        "frac_mfma_peak": round(entry_t / PEAK_TFLOPS[kernel_of(f)], 4),
                        "gbs": round(entry_gbs, 1), "frac_hbm_peak": round(entry_gbs / HBM_GBS, 4)})
        result["per_format"] = per
        result["peak_notes"] = PEAK_NOTE
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
