"""Parity of the square-tile small-cache backward (attn_bwd_smallcache) with
the float64 oracle's gradients.

The GPU path consumes the GPU forward's O and lse; the oracle computes the
exact gradients from Q, K, V, dO alone.  Small ragged shapes cover every
tile choice (b = 128 or 64, one or two staged panels) and are compared over
every element.  At full size, the d=256 backward workload (batch 1 x 8 heads,
N 4096) and the d=128 backward workload (2 x 16 heads, N 4096, run here at
M = 12288 < d^2) are compared on whole sampled heads and over every head
against sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.  Tolerance: max-abs 2e-2
(bf16 inputs and bf16 P / dS intermediates, fp32 accumulation).
"""
import pytest
import torch

import aware_tiling_amd as at
import oracle
from aware_tiling_amd.inputs import WORKLOADS
from tests.gpu_util import TOL, check, f64, inputs, say

pytestmark = pytest.mark.gpu

CASES = [
    # (bh, n, d, m_elems, seed, q_mult)
    (1, 64, 128, 12288, 301, 1.0),     # b 64, one stage
    (2, 200, 128, 12288, 302, 1.0),
    (1, 1, 128, 12288, 303, 1.0),
    (1, 257, 256, 49152, 304, 1.0),    # b 128, two stages
    (2, 130, 256, 40960, 305, 1.0),    # b 128, one stage
    (1, 300, 256, 16384, 306, 1.0),    # b 64, two stages
    (1, 100, 256, 12288, 307, 1.0),    # b 64, one stage
    (1, 513, 128, 12288, 308, 4.0),    # larger scores
    (1, 300, 256, 49152, 309, 20.0),   # peaked weights
]


def _grads(bh, n, d, seed, q_mult, m_elems):
    (qc, kc, vc, doc), (q, k, v, do) = inputs(bh, n, d, "bf16", seed, q_mult, with_do=True)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd(q, k, v, scale)
    dq, dk, dv = at.attn_bwd_smallcache(q, k, v, o, do, lse, m_elems, scale)
    torch.cuda.synchronize()
    return (qc, kc, vc, doc), (q, k, v, do, o, lse), (dq, dk, dv), scale


@pytest.mark.parametrize("bh,n,d,m_elems,seed,q_mult", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-M{c[3]}-q{c[5]:g}" for c in CASES])
def test_bwd_smallcache_matches_oracle(bh, n, d, m_elems, seed, q_mult):
    say(f"attn_bwd_smallcache bh={bh} n={n} d={d} M={m_elems} (b={at.bwd_smallcache_tile(d, m_elems)})"
        f" seed={seed} qx{q_mult}")
    (qc, kc, vc, doc), _, (dq, dk, dv), scale = _grads(bh, n, d, seed, q_mult, m_elems)
    rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc), f64(kc), f64(vc), f64(doc), scale)
    gs = q_mult > 1.0  # gradients grow with the scaled queries
    check(f64(dq), rq, TOL["bf16"], f"dQ {bh}x{n}x{d}/M{m_elems}", grad_scaled=gs)
    check(f64(dk), rk, TOL["bf16"], f"dK {bh}x{n}x{d}/M{m_elems}", grad_scaled=gs)
    check(f64(dv), rv, TOL["bf16"], f"dV {bh}x{n}x{d}/M{m_elems}", grad_scaled=gs)


@pytest.mark.parametrize("name,m_elems", [("bwd_smallcache_bf16_b1h8_n4096_d256", 49152),
                                          ("bwd_bf16_b2h16_n4096_d128", 12288)])
def test_bwd_smallcache_full_size(name, m_elems):
    w = WORKLOADS[name]
    say(f"attn_bwd_smallcache full workload {w.name} M={m_elems}")
    (qc, kc, vc, doc), (q, k, v, do, o, lse), (dq, dk, dv), scale = _grads(
        w.bh, w.n, w.d, w.seed, 1.0, m_elems)
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    sk = dk.double().sum(dim=1).abs().max().item()
    sv = (dv.double().sum(dim=1) - do.double().sum(dim=1)).abs().max().item()
    say(f"  max |sum_j dK_j| {sk:.3e}, max |sum_j dV_j - sum_i dO_i| {sv:.3e}")
    assert sk <= 5e-2 and sv <= 5e-2
    for h in (0, w.bh - 1):
        rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc[h:h + 1]), f64(kc[h:h + 1]), f64(vc[h:h + 1]),
                                           f64(doc[h:h + 1]), scale)
        check(f64(dq[h:h + 1]), rq, TOL["bf16"], f"dQ head {h}")
        check(f64(dk[h:h + 1]), rk, TOL["bf16"], f"dK head {h}")
        check(f64(dv[h:h + 1]), rv, TOL["bf16"], f"dV head {h}")


def test_bwd_smallcache_deterministic():
    _, (q, k, v, do, o, lse), (dq, dk, dv), scale = _grads(2, 333, 256, 310, 1.0, 49152)
    for _ in range(2):
        g = at.attn_bwd_smallcache(q, k, v, o, do, lse, 49152, scale)
        torch.cuda.synchronize()
        assert torch.equal(g[0], dq) and torch.equal(g[1], dk) and torch.equal(g[2], dv)


def test_bwd_smallcache_rejects_bad_budget():
    (_, (q, k, v, do)) = inputs(1, 64, 128, "bf16", 311, with_do=True)
    o, lse = at.attn_fwd(q, k, v)
    with pytest.raises(at.AttnError):
        at.attn_bwd_smallcache(q, k, v, o, do, lse, 128 * 128)  # not below d^2
    (_, (q2, k2, v2, do2)) = inputs(1, 64, 64, "bf16", 312, with_do=True)
    o2, lse2 = at.attn_fwd(q2, k2, v2)
    with pytest.raises(at.AttnError):
        at.attn_bwd_smallcache(q2, k2, v2, o2, do2, lse2, 4000)  # no tile fits
