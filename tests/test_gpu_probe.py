"""The benchmark-only MFMA probe on the GPU: the flop count is exact, the
clock it reports is a plausible shader clock, and the rate is positive and
below the device's dense bf16 peak at that clock (4096 flop per CU per cycle)."""

import numpy as np
import pytest
import torch

import lm_head_log_amd as lmh
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("operands", ["zeros", "random"])
def test_probe_rate_and_clock(operands):
    say(f"case: mfma probe, {operands} operands, 2000 iterations")
    dev = torch.device("cuda:0")
    if operands == "zeros":
        a = b = None
    else:
        g = torch.Generator(device="cpu").manual_seed(7)
        a = (torch.randn(1 << 20, generator=g) * 0.02).to(torch.bfloat16).to(dev)
        b = torch.randn(1 << 20, generator=g).to(torch.bfloat16).to(dev)
    r = lmh.lmhead_mfma_probe(a, b, 2000, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # per wave and iteration: 2 fragment sets x 64 MFMAs of 16 x 16 x 32
    flops = cus * 4 * 2000 * 2 * 64 * (2 * 16 * 16 * 32)
    assert r["ms"] > 0
    np.testing.assert_allclose(r["tflops"] * r["ms"] * 1e-3 * 1e12, flops, rtol=1e-9)
    assert 0.3 < r["clock_ghz"] < 3.5, r
    # no more than the dense peak at the reported clock (small slack: the
    # clock is averaged over each workgroup's loop, the time over the launch)
    assert r["tflops"] <= cus * 4096 * r["clock_ghz"] * 1e9 / 1e12 * 1.05, r


def test_probe_rejects_one_operand():
    dev = torch.device("cuda:0")
    a = torch.zeros(64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        lmh.lmhead_mfma_probe(a, None, 10)
