"""The allocation-free key-split forward (attn_fwd_splitk_noalloc) against
the workspace form (attn_fwd_splitk) and the float64 oracle.

Two calls in a row, the second with a smaller input, so the second reuses
the library's device array with the first call's partials still in it; each
call is compared with attn_fwd_splitk on the same inputs (the same kernels,
so bit for bit) and with the oracle (max-abs 2e-2, bf16 inputs).  A single
chunk (no partials) and a request too large for the array are covered too.
"""
import pytest
import torch

import aware_tiling_amd as at
import oracle
from aware_tiling_amd.inputs import make_inputs
from tests.gpu_util import TOL, check, f64, say

pytestmark = pytest.mark.gpu


def _case(bh, nq, nk, d, splits, seed, q_mult=1.0):
    qc, kc, vc = make_inputs(bh, nq, d, "bf16", seed, q_mult, nk=nk)
    q, k, v = (t.to("cuda") for t in (qc, kc, vc))
    scale = at.default_scale(d)
    out = torch.full((bh, nq, d), float("nan"), device="cuda")
    lse = torch.full((bh, nq), float("nan"), device="cuda")
    at.attn_fwd_splitk_noalloc(q, k, v, out, lse, splits, scale)
    ref_o, ref_l = at.attn_fwd_splitk(q, k, v, splits, scale)
    torch.cuda.synchronize()
    used = at.splitk_splits(bh, nq, nk, d, splits)
    say(f"attn_fwd_splitk_noalloc bh={bh} nq={nq} nk={nk} d={d} splits={splits} (uses {used})")
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "differs from attn_fwd_splitk"
    ro, rl, _ = oracle.attn_fwd(f64(qc), f64(kc), f64(vc), scale)
    check(f64(out), ro, TOL["bf16"], "O no-alloc")
    check(f64(lse), rl, TOL["bf16"], "lse no-alloc")
    return used


def test_noalloc_two_calls_second_smaller():
    # decoding-like: one query per head, automatic chunking
    assert _case(64, 1, 5000, 128, 0, 301) > 1
    # smaller, different d and chunk count, peaked weights: every partial
    # the first call left in the array must be overwritten or unused
    assert _case(3, 37, 777, 64, 5, 302, 8.0) > 1


def test_noalloc_single_chunk_and_too_large_request():
    assert _case(2, 200, 150, 128, 1, 303) == 1
    bh, nq, nk, d, splits = 64, 200, 4096, 128, 16
    need = int(at.lib().attn_fwd_splitk_workspace_size(bh, nq, nk, d, splits))
    assert need > at.binding.SPLITK_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((bh, nq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((bh, nk, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((bh, nq, d), device="cuda")
    with pytest.raises(at.AttnError, match="WORKSPACE"):
        at.attn_fwd_splitk_noalloc(q, kv, kv, out, None, splits)
