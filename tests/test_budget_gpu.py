"""Parity of the fused forward held to an on-chip budget below d^2
(attn_fwd_budget: 32-row query blocks, 32-key tiles, four waves splitting d).

It computes the same function as the definition, so it is compared with
the float64 oracle over every element on small ragged shapes (tails in both
the query blocks and the key tiles, one row, peaked weights), on sampled
rows at the batch 1 x 8 heads, N 4096, d 256 size, and everywhere against
attn_fwd and attn_fwd_smallcache run on the same inputs at the same budget.
Tolerance: max-abs 2e-2 (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import aware_tiling_amd as at
from aware_tiling_amd.inputs import WORKLOADS
from tests.gpu_util import (TOL, check, f64, gather_rows, inputs, oracle_fwd_head_rows,
                            oracle_fwd_rows, rows_every_block, say)

pytestmark = pytest.mark.gpu

CASES = [
    # (bh, n, d, seed, q_mult)
    (1, 1, 256, 501, 1.0),
    (2, 33, 256, 502, 1.0),
    (1, 300, 256, 503, 1.0),
    (3, 257, 128, 504, 1.0),
    (1, 640, 256, 505, 4.0),
    (1, 200, 256, 506, 40.0),  # scores in the hundreds: every tile rescales
]


@pytest.mark.parametrize("bh,n,d,seed,q_mult", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-q{c[4]:g}" for c in CASES])
def test_budget_matches_oracle(bh, n, d, seed, q_mult):
    m = at.fwd_budget_onchip_elems(d)
    say(f"attn_fwd_budget bh={bh} n={n} d={d} M={m} seed={seed} qx{q_mult}")
    (qc, kc, vc), (q, k, v) = inputs(bh, n, d, "bf16", seed, q_mult)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd_budget(q, k, v, m, scale)
    torch.cuda.synchronize()
    ro, rl = oracle_fwd_rows(qc, kc, vc, scale, np.arange(bh), np.arange(n))
    check(f64(o), ro, TOL["bf16"], f"O budget {bh}x{n}x{d}")
    check(f64(lse), rl, TOL["bf16"], f"lse budget {bh}x{n}x{d}")


def test_budget_full_size_against_oracle_and_other_paths():
    w = WORKLOADS["smallcache_bf16_b1h8_n4096_d256"]
    m = at.fwd_budget_onchip_elems(w.d)
    assert m < w.d * w.d
    say(f"attn_fwd_budget full workload {w.name} M={m} (small-cache tile b="
        f"{at.smallcache_tile(w.d, m)} at the same M)")
    (qc, kc, vc), (q, k, v) = inputs(w.bh, w.n, w.d, w.dtype, w.seed, w.q_mult)
    o, lse = at.attn_fwd_budget(q, k, v, m, w.scale)
    o2, lse2 = at.attn_fwd_budget(q, k, v, m, w.scale)
    of, lf = at.attn_fwd(q, k, v, w.scale)
    osc, lsc = at.attn_fwd_smallcache(q, k, v, m, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    # one row from every (head, 32-row query block): every workgroup
    rows = rows_every_block(w.bh, w.n, 32, 1, w.seed)
    ro, rl = oracle_fwd_head_rows(qc, kc, vc, w.scale, rows)
    check(gather_rows(o, rows), ro, TOL["bf16"], "O budget every block")
    check(gather_rows(lse, rows), rl, TOL["bf16"], "lse budget every block")
    for other, lo, name in ((of, lf, "attn_fwd"), (osc, lsc, "attn_fwd_smallcache")):
        diff = float((o - other).abs().max())
        ldiff = float((lse - lo).abs().max())
        say(f"  max |O_budget - O_{name}| {diff:.3e}, max |lse diff| {ldiff:.3e}")
        assert diff <= 2 * TOL["bf16"] and ldiff <= 2 * TOL["bf16"]


def test_budget_rejects_too_small_budget():
    (_, (q, k, v)) = inputs(1, 64, 256, "bf16", 507)
    with pytest.raises(at.AttnError):
        at.attn_fwd_budget(q, k, v, at.fwd_budget_onchip_elems(256) - 1)
