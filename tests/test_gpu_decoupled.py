"""GPU parity of the BF16 kernel with decoupled A / B rings
(gemm_bf16_decoupled) through the C ABI, with A's slot released early and
at the stage's end: against the oracle, and bit for bit against gemm_bf16
(both accumulate the k-steps in the same order).  The shapes cover the A
stream running a whole tile ahead (two stages a tile) and one stage into the
next tile (three), more tiles than CUs (a second persistent round), ragged M
and N, a partial last stage, and few tiles."""
import numpy as np
import pytest
import torch

import dense_block_scaled_amd as dbs
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

RELEASE = [True, False]


def _rid(e):
    return "early-A" if e else "late-A"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)


SHAPES = [
    (2304, 2304, 1024),     # 81 tiles, 16 stages
    (4352, 4352, 128),      # 289 tiles, 2 stages: the early A stream a whole tile ahead
    (4352, 4352, 192),      # 289 tiles, 3 stages
    (2200, 2600, 328),      # ragged tiles, partial last stage (K % 64 == 8)
    (300, 520, 136),        # 6 tiles, 3 stages, partial last stage
    (4096, 4096, 4096),     # one persistent round of 256 tiles, 64 stages
]


@pytest.mark.parametrize("early", RELEASE, ids=_rid)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decoupled_matches_oracle_and_gemm_bf16(shape, early):
    M, N, K = shape
    _gpu.say(f"[decoupled] {_rid(early)} {shape}")
    w = synth.workload("bf16", M, N, K, 600 + M % 17, 610 + N % 19)
    d = _gpu.to_dev(w)
    D = dbs.gemm_bf16_decoupled(d["A"], d["B"], early_release_a=early)
    R = dbs.gemm_bf16(d["A"], d["B"])
    torch.cuda.synchronize()
    if M * N <= 6 << 20:
        _gpu.check_full("bf16", w, D)
    else:
        em, en = synth.sample_entries(85, M, N, 4096)
        _gpu.check_sampled("bf16", w, D, em, en)
    assert torch.equal(D.view(torch.int16), R.view(torch.int16)), "differs from gemm_bf16"


@pytest.mark.parametrize("early", RELEASE, ids=_rid)
def test_decoupled_exact_permutation(early):
    """A times a permutation matrix: every output is one element of A."""
    M, K = 2304, 2304
    _gpu.say(f"[decoupled] {_rid(early)} exact permutation")
    rng = np.random.default_rng(86)
    w = synth.workload("bf16", M, K, K, 620, 621)
    eye = np.zeros((K, K), np.float32)
    eye[np.arange(K), rng.permutation(K)] = 1.0
    w["B"] = synth.bf16_from_f32(eye)
    d = _gpu.to_dev(w)
    D = dbs.gemm_bf16_decoupled(d["A"], d["B"], early_release_a=early)
    torch.cuda.synchronize()
    em, en = synth.sample_entries(87, M, K, 4096)
    _gpu.check_exact_sampled("bf16", w, D, em, en)


@pytest.mark.parametrize("early", RELEASE, ids=_rid)
def test_decoupled_repeats_bitwise(early):
    """Ten launches in a row on one stream give the same bits."""
    M, N, K = 4352, 4352, 192
    _gpu.say(f"[decoupled] {_rid(early)} repeats")
    w = synth.workload("bf16", M, N, K, 630, 631)
    d = _gpu.to_dev(w)
    first = dbs.gemm_bf16_decoupled(d["A"], d["B"], early_release_a=early).clone()
    for _ in range(9):
        D = dbs.gemm_bf16_decoupled(d["A"], d["B"], early_release_a=early)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), D.view(torch.int16))
