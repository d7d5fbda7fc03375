"""Parity of the square-tile small-cache forward (attn_fwd_smallcache).

The square-tile schedule reaches the same function as the definition (it only
keeps the exponentiated score matrix in device memory), so it is compared
with the float64 oracle of the definition: in full on small ragged shapes,
on rows from every (head, query tile) at the full batch 1 x 8 heads,
N 4096, d 256 size, and
against the fused path on the same inputs.  Tolerance: max-abs 2e-2 (bf16).
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
    # (bh, n, d, m_elems, seed, q_mult)
    (1, 300, 256, 49152, 61, 1.0),  # b = 128
    (2, 300, 256, 40000, 62, 1.0),  # b = 64
    (1, 1, 256, 49152, 63, 1.0),
    (2, 17, 256, 49152, 64, 1.0),
    (1, 513, 256, 49152, 65, 4.0),
    (3, 200, 128, 16000, 66, 1.0),  # d = 128 -> b = 64
    (1, 257, 128, 12288, 67, 1.0),  # budget = the b = 64 footprint
    (1, 640, 256, 49152, 68, 40.0),  # scores in the hundreds
]


@pytest.mark.parametrize("bh,n,d,m_elems,seed,q_mult", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-M{c[3]}-q{c[5]:g}" for c in CASES])
def test_smallcache_matches_oracle(bh, n, d, m_elems, seed, q_mult):
    b = at.smallcache_tile(d, m_elems)
    say(f"attn_fwd_smallcache bh={bh} n={n} d={d} M={m_elems} b={b} qx{q_mult}")
    assert b > 0
    (qc, kc, vc), (q, k, v) = inputs(bh, n, d, "bf16", seed, q_mult)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd_smallcache(q, k, v, m_elems, scale)
    torch.cuda.synchronize()
    ro, rl = oracle_fwd_rows(qc, kc, vc, scale, np.arange(bh), np.arange(n))
    check(f64(o), ro, TOL["bf16"], f"O smallcache {bh}x{n}x{d} b{b}")
    check(f64(lse), rl, TOL["bf16"], f"lse smallcache {bh}x{n}x{d} b{b}")


def test_smallcache_full_size_against_oracle_and_fused():
    w = WORKLOADS["smallcache_bf16_b1h8_n4096_d256"]
    m_elems = 49152
    say(f"attn_fwd_smallcache full workload {w.name} M={m_elems}")
    (qc, kc, vc), (q, k, v) = inputs(w.bh, w.n, w.d, w.dtype, w.seed, w.q_mult)
    o, lse = at.attn_fwd_smallcache(q, k, v, m_elems, w.scale)
    of, lf = at.attn_fwd(q, k, v, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # rows from every (head, query tile of b rows): every output tile of the
    # value product and every query block of the fused kernel
    b = at.smallcache_tile(w.d, m_elems)
    rows = rows_every_block(w.bh, w.n, b, 2, w.seed)
    say(f"  oracle on {rows.size} rows: 2 from each of {w.bh} heads x {w.n // b} tiles of {b}")
    ro, rl = oracle_fwd_head_rows(qc, kc, vc, w.scale, rows)
    check(gather_rows(o, rows), ro, TOL["bf16"], "O smallcache every tile")
    check(gather_rows(lse, rows), rl, TOL["bf16"], "lse smallcache every tile")
    check(gather_rows(of, rows), ro, TOL["bf16"], "O fused every tile (same inputs)")
    # both paths compute the same function: compare them everywhere
    diff = float((o - of).abs().max())
    say(f"  max |O_smallcache - O_fused| over all elements: {diff:.3e}")
    assert diff <= 2 * TOL["bf16"]
    ldiff = float((lse - lf).abs().max())
    say(f"  max |lse_smallcache - lse_fused|: {ldiff:.3e}")
    assert ldiff <= 2 * TOL["bf16"]


def test_smallcache_deterministic_and_workspace_reuse():
    (_, (q, k, v)) = inputs(2, 700, 256, "bf16", 69)
    need = int(at.lib().attn_fwd_smallcache_workspace_size(2, 700, 256, 49152))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # garbage contents
    o1, l1 = at.attn_fwd_smallcache(q, k, v, 49152, workspace=ws)
    o2, l2 = at.attn_fwd_smallcache(q, k, v, 49152, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_smallcache_rejects_small_workspace_and_large_budget():
    (_, (q, k, v)) = inputs(1, 64, 256, "bf16", 70)
    need = int(at.lib().attn_fwd_smallcache_workspace_size(1, 64, 256, 49152))
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(at.AttnError):
        at.attn_fwd_smallcache(q, k, v, 49152, workspace=ws)
    with pytest.raises(at.AttnError):
        at.attn_fwd_smallcache(q, k, v, 256 * 256)
