"""GPU check of gemm_nvfp4_fp8_noalloc through the C ABI: bit for bit the
result of gemm_nvfp4_fp8 with a caller workspace, on two calls in a row, the
second on a smaller problem (the static workspace keeps the first call's
contents), and within the FP8-rate oracle's tolerance."""
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


def _pair(M, N, K, seed):
    w = synth.workload("nvfp4", M, N, K, seed, seed + 1)
    d = _gpu.to_dev(w)
    ws = torch.empty(dbs.nvfp4_fp8_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    want = dbs.gemm_nvfp4_fp8(d["A"], d["sA"], w["tA"], d["B"], d["sB"], w["tB"], workspace=ws)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    got = dbs.gemm_nvfp4_fp8_noalloc(d["A"], d["sA"], w["tA"], d["B"], d["sB"], w["tB"], out=out)
    torch.cuda.synchronize()
    return w, want, got


def test_noalloc_matches_caller_workspace_twice():
    for (M, N, K), seed in (((640, 520, 2048), 71), ((300, 200, 512), 73)):
        _gpu.say(f"[noalloc] {M}x{N}x{K}")
        w, want, got = _pair(M, N, K, seed)
        assert torch.equal(want.view(torch.int16), got.view(torch.int16))
        wq = oracle.nvfp4_fp8_workload(w)
        d, an, bn = oracle.gemm_full("mxfp8", wq)
        alpha = float(w["tA"]) * float(w["tB"])
        r = oracle.rel_errors(_gpu.d_to_numpy(got), d * alpha, an * abs(alpha), bn)
        assert np.all(np.isfinite(r)) and float(r.max()) <= _gpu.tol_bound(K)


def test_noalloc_rejects_problems_beyond_its_workspace():
    M, N, K = 4096, 4096, 8192          # 69 MB of workspace, above the static 64 MiB
    assert dbs.nvfp4_fp8_workspace_bytes(M, N, K) > 64 << 20
    A = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((M, K // 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dbs.DbsError) as e:
        dbs.gemm_nvfp4_fp8_noalloc(A, s, 1.0, A, s, 1.0, out=out)
    assert e.value.status == dbs.DBS_EINVAL and "workspace" in str(e.value)
