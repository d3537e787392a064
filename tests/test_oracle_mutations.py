"""Planted mistakes in the oracle (on the CPU) must each be caught by a pin.

Not listed: swapping the FP4 nibble order.  Applied to both operands it
permutes k identically inside one scale block (k and k^1 share a block), so
every dot product -- hence D -- is unchanged; it is unobservable in the GEMM.
The packing convention (element 2j in the low nibble) is instead checked where
it is observable, in the quantiser cross-check of tests/test_synth.py.
"""
import pytest

import oracle
from tests import _pins

MUTATIONS = {
    2: "scale of the next block applied",
    3: "NVFP4 tensor scales dropped",
    4: "A*B instead of A*B^T",
    5: "E4M3 exponent bias 8",
    6: "E2M1 subnormal decoded as 1.0",
    7: "fp32 accumulation",
    8: "E8M0 bias 128",
    9: "last K term dropped",
    10: "E4M3 sign ignored",
    11: "bf16 mantissa truncated",
    12: "E5M2 exponent bias 16",
    13: "E5M2 subnormals read as normals",
}


def test_unmutated_battery_passes():
    res = _pins.battery()
    assert all(res.values()), [k for k, v in res.items() if not v]


@pytest.mark.parametrize("mut", sorted(MUTATIONS))
def test_each_planted_mistake_is_caught(mut):
    oracle.set_mutation(mut)
    try:
        res = _pins.battery()
    finally:
        oracle.set_mutation(0)
    failed = [k for k, v in res.items() if not v]
    assert failed, f"planted mistake '{MUTATIONS[mut]}' passed every pin"
