"""GPU parity at the benchmark workloads, in the launch configuration the
benchmark times (same entry points, same grid logic).

* BF16 4096^3: every output against the oracle.
* BF16/MXFP8/MXFP4/NVFP4 8192^3, MXFP4 16384^3 and NVFP4 256x16384x8192:
  4096 seeded output entries (the rows/columns {0, 255, 256, last} crossed,
  then uniform draws) against the oracle, one by one.

Seeds follow the workload index c: A from 100c+1, B from 100c+2, sampled
entries from 100c+3 (c = 1 bf16, 2 mxfp8, 3 mxfp4, 4 nvfp4).
"""
import pytest
import torch

import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


def _run_sampled(fmt, c, M, N, K):
    _gpu.say(f"[config] {fmt} {M}x{N}x{K} (seeds {100 * c + 1}, {100 * c + 2}, {100 * c + 3})")
    w = synth.workload(fmt, M, N, K, 100 * c + 1, 100 * c + 2)
    D = _gpu.run(fmt, w)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(100 * c + 3, M, N, 4096)
    return _gpu.check_sampled(fmt, w, D, em, en)


@pytest.mark.timeout(300)
def test_bf16_4096_full():
    _gpu.say("[config] bf16 4096^3 full")
    w = synth.workload("bf16", 4096, 4096, 4096, 101, 102)
    D = _gpu.run("bf16", w)
    torch.cuda.synchronize()
    _gpu.check_full("bf16", w, D)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("fmt,c", [("bf16", 1), ("mxfp8", 2), ("mxfp4", 3), ("nvfp4", 4)])
def test_8192_cube_sampled(fmt, c):
    _run_sampled(fmt, c, 8192, 8192, 8192)


@pytest.mark.timeout(600)
def test_mxfp4_16384_cube_sampled():
    _run_sampled("mxfp4", 3, 16384, 16384, 16384)


@pytest.mark.timeout(300)
def test_nvfp4_skinny_sampled():
    _run_sampled("nvfp4", 4, 256, 16384, 8192)
