"""Host logic of bench.py, no GPU: the one-GPU guard, the algorithmic byte
counts the roofline divides by, the per-workload record's fractions, the
traffic lookup's source-hash rule and the provenance fields."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,want", [
    # A and B at the element width, their scale bytes (one per block), D in bf16
    ("bf16", 2 * 8192 * 8192 * 2 + 8192 * 8192 * 2),
    ("mxfp8", 2 * 8192 * 8192 + 2 * 8192 * 8192 // 32 + 8192 * 8192 * 2),
    ("mxfp4", 2 * 8192 * 8192 // 2 + 2 * 8192 * 8192 // 32 + 8192 * 8192 * 2),
    ("nvfp4", 2 * 8192 * 8192 // 2 + 2 * 8192 * 8192 // 16 + 8192 * 8192 * 2),
    ("nvfp4_skinny", (256 + 16384) * 8192 // 2 + (256 + 16384) * 8192 // 16 + 256 * 16384 * 2),
])
def test_algorithmic_bytes(name, want):
    M, N, K = bench.W[name]["shape"]
    assert bench.algorithmic_bytes(name, M, N, K) == want


def test_record_prices_each_line_at_its_own_peak():
    M, N, K = bench.W["nvfp4_skinny"]["shape"]
    avg = 80e-6
    tflops = 2.0 * M * N * K / avg / 1e12
    e = bench.record("nvfp4_skinny", {"M": M, "N": N, "K": K}, avg, tflops, 1000.0, 2000.0, 1e-4, None)
    assert e["peak_tflops"] == 2500.0 and e["frac_mfma_peak"] == round(tflops / 2500.0, 4)
    assert e["frac_fp4_peak"] == round(tflops / 10100.0, 4)
    assert e["frac_mfma_peak_at_sclk"] == round(tflops / (2500.0 * 2000.0 / bench.CLOCK_PEAK_MHZ), 4)
    # the skinny line's path roofline: the larger of its HBM time and its fp16 MFMA time, over the launch time
    t_min = max(bench.algorithmic_bytes("nvfp4_skinny", M, N, K) / 8e12, 2.0 * M * N * K / 2.5e15)
    assert e["frac_path_roofline"] == round(t_min / avg, 4)
    assert e["seeds"] == {"A": 401, "B": 402, "sampled_entries": 403}
    e6 = bench.record("mx_e2m3_e2m3", {"M": 8192, "N": 8192, "K": 8192}, 5e-4, 2200.0, 500.0, None, 1e-4, None)
    assert e6["peak_tflops"] == 10100.0 and e6["sclk_mhz"] is None


def test_traffic_lookup_follows_the_source_hash(monkeypatch):
    d = json.loads((ROOT / "profiles" / "traffic.json").read_text())
    names = list(d["workloads"])
    assert "bf16_gemm_8192x8192x8192" in names
    if d["kernel_source_sha"] == bench.kernel_source_hash():
        for n in names:
            assert bench.traffic_for(n) == d["workloads"][n]["hbm_bytes_per_launch"] > 0
    assert bench.traffic_for("no_such_workload") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert all(bench.traffic_for(n) is None for n in names)


def test_provenance():
    p = bench.provenance("mxfp4")
    assert p["seeds"] == {"A": 301, "B": 302, "sampled_entries": 303}
    assert p["kernel_source_sha"] == bench.kernel_source_hash()
    r = subprocess.run(["git", "-C", str(ROOT), "rev-parse", "HEAD"], capture_output=True, text=True)
    if r.returncode == 0:
        assert p["git_sha"] == r.stdout.strip()
