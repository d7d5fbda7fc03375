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


def test_calib_stream_read_xor_per_thread():
    """Thread t's word is the XOR of the 32-bit words of the 16-byte chunks
    t, t + T, t + 2T, ... of the buffer (T threads), computed here on the
    host; a ragged last round (chunks not a multiple of T) included."""
    wgs = 3
    threads = wgs * 256
    chunks = 5 * threads + 77
    g = torch.Generator().manual_seed(5)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (chunks * 4,), dtype=torch.int64,
                         generator=g).to(torch.int32)
    say(f"attn_calib_stream_read {chunks} chunks over {threads} threads")
    src = host.to("cuda")
    out = torch.zeros(threads, dtype=torch.int32, device="cuda")
    assert at.calib_stream_read(src, out) == chunks * 16
    torch.cuda.synchronize()
    words = host.view(chunks, 4).numpy().astype("uint32")
    want = [0] * threads
    for i in range(chunks):
        w = words[i]
        want[i % threads] ^= int(w[0] ^ w[1] ^ w[2] ^ w[3])
    got = out.cpu().numpy().astype("uint32").tolist()
    assert got == want
