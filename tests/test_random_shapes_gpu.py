"""Seeded random shapes through every entry point, against the float64 oracle.

Each case draws bh in {1, 2, 3}, N from a list of ragged lengths (1, tile
boundaries plus and minus one, non-powers of two), d in {64, 128, 256} and
a query scale of 1 or 4, then runs whichever of attn_fwd, attn_fwd_budget,
attn_fwd_smallcache, attn_fwd_splitk, attn_fwd_blocksparse, attn_bwd and
attn_bwd_smallcache support that d, each compared over every element.
Tolerance: max-abs 2e-2 (bf16 inputs) for O and lse at every query scale;
gradients of the x4 cases relative to max(1, max|ref|), as in the other
backward tests.
"""
import random

import numpy as np
import pytest
import torch

import aware_tiling_amd as at
import oracle
from aware_tiling_amd.inputs import make_block_mask
from tests.gpu_util import TOL, check, f64, inputs, say

pytestmark = pytest.mark.gpu

LENGTHS = [1, 2, 31, 33, 63, 65, 100, 127, 129, 200, 255, 257, 300, 511, 640]


def _case(i):
    rng = random.Random(7000 + i)
    return (rng.choice([1, 2, 3]), rng.choice(LENGTHS), rng.choice([64, 128, 256]),
            rng.choice([1.0, 4.0]), rng.choice([0, 1, 2, 5]), rng.choice([1, 3, 64, 129]),
            rng.random() < 0.5)


CASES = [_case(i) for i in range(24)]


@pytest.mark.parametrize("i", range(len(CASES)),
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-q{c[3]:g}" for c in CASES])
def test_random_shape_all_paths(i):
    bh, n, d, qm, splits, nq, diag = CASES[i]
    seed = 7000 + i
    say(f"random shape {i}: bh={bh} n={n} d={d} qx{qm} seed={seed}")
    (qc, kc, vc, doc), (q, k, v, do) = inputs(bh, n, d, "bf16", seed, qm, with_do=True)
    s = at.default_scale(d)
    gs = qm > 1.0  # gradients grow with the scaled queries; O and lse do not
    ro, rl, _ = oracle.attn_fwd(f64(qc), f64(kc), f64(vc), s)
    o, lse = at.attn_fwd(q, k, v, s)
    torch.cuda.synchronize()
    check(f64(o), ro, TOL["bf16"], "attn_fwd O")
    check(f64(lse), rl, TOL["bf16"], "attn_fwd lse")
    if d in (128, 256):
        ob, _ = at.attn_fwd_budget(q, k, v, at.fwd_budget_onchip_elems(d), s)
        torch.cuda.synchronize()
        check(f64(ob), ro, TOL["bf16"], "attn_fwd_budget O")
        for m in (12288, 49152):
            if at.smallcache_tile(d, m) > 0:
                osc, lsc = at.attn_fwd_smallcache(q, k, v, m, s)
                torch.cuda.synchronize()
                check(f64(osc), ro, TOL["bf16"], f"attn_fwd_smallcache M{m} O")
                check(f64(lsc), rl, TOL["bf16"], f"attn_fwd_smallcache M{m} lse")
    if d in (64, 128, 256):
        nqq = min(nq, n)
        osk, _ = at.attn_fwd_splitk(q[:, :nqq].contiguous(), k, v, splits, s)
        torch.cuda.synchronize()
        check(f64(osk), ro[:, :nqq], TOL["bf16"], f"attn_fwd_splitk({splits}) O")
        mask = make_block_mask(bh, -(-n // at.SPARSE_BLOCK), 0.5, seed, keep_diagonal=diag)
        osp, lsp = at.attn_fwd_blocksparse(q, k, v, mask.to("cuda"), s)
        torch.cuda.synchronize()
        rm, rml, _ = oracle.attn_fwd_masked(f64(qc), f64(kc), f64(vc), s, mask.numpy(),
                                            at.SPARSE_BLOCK, at.SPARSE_BLOCK)
        empty = np.isneginf(rml)
        assert np.array_equal(np.isneginf(f64(lsp)), empty)
        check(f64(osp), rm, TOL["bf16"], "attn_fwd_blocksparse O")
    if n <= 300 and d in (64, 128, 256):
        rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc), f64(kc), f64(vc), f64(doc), s)
        grads = []
        grads.append(("attn_bwd", at.attn_bwd(q, k, v, o, do, lse, s)))
        if at.bwd_smallcache_tile(d, 12288) > 0:
            grads.append(("attn_bwd_smallcache", at.attn_bwd_smallcache(q, k, v, o, do, lse,
                                                                        12288, s)))
        torch.cuda.synchronize()
        for name, (dq, dk, dv) in grads:
            check(f64(dq), rq, TOL["bf16"], f"{name} dQ", grad_scaled=gs)
            check(f64(dk), rk, TOL["bf16"], f"{name} dK", grad_scaled=gs)
            check(f64(dv), rv, TOL["bf16"], f"{name} dV", grad_scaled=gs)
