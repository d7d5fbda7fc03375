"""The calibration matrix-core loop (attn_calib_mfma_loop): with zero
operands every accumulator stays exactly 0; with random operands the
per-thread sums are finite and the launch is repeatable bit for bit.
Not part of the attention method; it gives bench.py a reachable MFMA rate."""
import pytest
import torch

import aware_tiling_amd as at
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_calib_mfma_loop_zero_and_random():
    say("attn_calib_mfma_loop 8 workgroups x 50 rounds")
    out = torch.full((8 * 256,), 7.0, dtype=torch.float32, device="cuda")
    flops = at.calib_mfma_loop(out, 50, 0.0)
    torch.cuda.synchronize()
    assert flops == 8 * 50 * 4 * 4 * 2 * 32 * 32 * 16
    assert torch.count_nonzero(out).item() == 0
    at.calib_mfma_loop(out, 50, 1.0)
    first = out.clone()
    at.calib_mfma_loop(out, 50, 1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(first).all() and torch.count_nonzero(first).item() > 0
    assert torch.equal(first, out)
