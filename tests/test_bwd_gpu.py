"""Parity of the backward (attn_bwd) with the float64 oracle's gradients.

The GPU backward consumes the GPU forward's O and lse (end to end); the
oracle computes the exact gradients from Q, K, V, dO alone.  Small ragged
shapes are compared over every element; the full batch 2 x 16 heads,
N 4096, d 128 workload is compared on whole sampled heads (dK and dV of a
key need every query, so sampling is by head), and over every head against
two identities that hold at any size: sum_j dK_j = 0 (a common shift of all
keys changes no weight) and sum_j dV_j = sum_i dO_i (each row of weights
sums to one).  Tolerance: max-abs 2e-2 (bf16 inputs, fp32 accumulation).
"""
import pytest
import torch

import aware_tiling_amd as at
import oracle
from aware_tiling_amd.inputs import WORKLOADS
from tests.gpu_util import TOL, check, f64, inputs, say

pytestmark = pytest.mark.gpu

CASES = [
    # (bh, n, d, seed, q_mult)
    (1, 64, 64, 81, 1.0),
    (2, 200, 128, 82, 1.0),
    (1, 257, 64, 83, 1.0),
    (1, 1, 128, 84, 1.0),
    (2, 17, 128, 85, 1.0),
    (1, 513, 128, 86, 4.0),
    (1, 300, 128, 87, 20.0),  # peaked weights
    (3, 160, 64, 88, 1.0),
    (1, 200, 256, 92, 1.0),
    (2, 129, 256, 93, 4.0),
    (1, 1, 256, 94, 1.0),
]


def _grads(bh, n, d, seed, q_mult):
    (qc, kc, vc, doc), (q, k, v, do) = inputs(bh, n, d, "bf16", seed, q_mult, with_do=True)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd(q, k, v, scale)
    dq, dk, dv = at.attn_bwd(q, k, v, o, do, lse, scale)
    torch.cuda.synchronize()
    return (qc, kc, vc, doc), (q, k, v, do), (dq, dk, dv), scale


@pytest.mark.parametrize("bh,n,d,seed,q_mult", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-q{c[4]:g}" for c in CASES])
def test_bwd_matches_oracle(bh, n, d, seed, q_mult):
    say(f"attn_bwd bh={bh} n={n} d={d} seed={seed} qx{q_mult}")
    (qc, kc, vc, doc), _, (dq, dk, dv), scale = _grads(bh, n, d, seed, q_mult)
    rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc), f64(kc), f64(vc), f64(doc), scale)
    gs = q_mult > 1.0  # gradients grow with the scaled queries
    check(f64(dq), rq, TOL["bf16"], f"dQ {bh}x{n}x{d}", grad_scaled=gs)
    check(f64(dk), rk, TOL["bf16"], f"dK {bh}x{n}x{d}", grad_scaled=gs)
    check(f64(dv), rv, TOL["bf16"], f"dV {bh}x{n}x{d}", grad_scaled=gs)


def test_bwd_full_size_sampled_heads_and_identities():
    w = WORKLOADS["bwd_bf16_b2h16_n4096_d128"]
    say(f"attn_bwd full workload {w.name}")
    (qc, kc, vc, doc), (q, k, v, do), (dq, dk, dv), scale = _grads(w.bh, w.n, w.d, w.seed, 1.0)
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    # identities over every head
    sk = dk.double().sum(dim=1).abs().max().item()
    sv = (dv.double().sum(dim=1) - do.double().sum(dim=1)).abs().max().item()
    say(f"  max |sum_j dK_j| {sk:.3e}, max |sum_j dV_j - sum_i dO_i| {sv:.3e}")
    assert sk <= 5e-2 and sv <= 5e-2
    # every head against the oracle (dK and dV of a key need every query, so
    # whole heads are compared; all of them, i.e. every workgroup's output)
    say(f"  oracle gradients for all {w.bh} heads")
    rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc), f64(kc), f64(vc), f64(doc), scale)
    check(f64(dq), rq, TOL["bf16"], "dQ all heads")
    check(f64(dk), rk, TOL["bf16"], "dK all heads")
    check(f64(dv), rv, TOL["bf16"], "dV all heads")


def test_bwd_deterministic():
    _, (q, k, v, do), (dq, dk, dv), scale = _grads(2, 333, 128, 89, 1.0)
    o, lse = at.attn_fwd(q, k, v, scale)
    for _ in range(3):
        g = at.attn_bwd(q, k, v, o, do, lse, scale)
        torch.cuda.synchronize()
        assert torch.equal(g[0], dq) and torch.equal(g[1], dk) and torch.equal(g[2], dv)


def test_bwd_rejects_unsupported_head_dim():
    (_, (q, k, v, do)) = inputs(1, 64, 96, "bf16", 90, with_do=True)
    o = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.zeros(q.shape[:2], dtype=torch.float32, device=q.device)
    with pytest.raises(at.AttnError):
        at.attn_bwd(q, k, v, o, do, lse)


def test_bwd_d256_workload_every_head():
    """The blockwise backward at d = 256 (four waves, 128 keys or queries
    per workgroup) on the batch 1 x 8 heads, N 4096 workload of the
    small-cache backward, every head against the oracle, and against the
    small-cache backward's gradients on the same inputs."""
    w = WORKLOADS["bwd_smallcache_bf16_b1h8_n4096_d256"]
    say(f"attn_bwd d=256 on {w.name}")
    (qc, kc, vc, doc), (q, k, v, do), (dq, dk, dv), scale = _grads(w.bh, w.n, w.d, w.seed, 1.0)
    rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc), f64(kc), f64(vc), f64(doc), scale)
    check(f64(dq), rq, TOL["bf16"], "dQ d256 all heads")
    check(f64(dk), rk, TOL["bf16"], "dK d256 all heads")
    check(f64(dv), rv, TOL["bf16"], "dV d256 all heads")


BWD_TILE_CASES = [(2, 300, 128, 89, 1.0), (1, 1000, 128, 90, 4.0), (1, 33, 128, 91, 1.0)]


@pytest.mark.parametrize("bh,n,d,seed,q_mult", BWD_TILE_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-q{c[4]:g}" for c in BWD_TILE_CASES])
def test_bwd_every_tile_shape_gives_the_default_bits(bh, n, d, seed, q_mult):
    """Every compiled backward tile shape (attn_bwd_tile) processes each
    wave's 32 rows in the same order as the default, so its gradients equal
    attn_bwd's bit for bit; the default is held to the oracle above."""
    (qc, kc, vc, doc), (q, k, v, do) = inputs(bh, n, d, "bf16", seed, q_mult, with_do=True)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd(q, k, v, scale)
    ref = at.attn_bwd(q, k, v, o, do, lse, scale)
    tiles = at.bwd_tiles(d)
    assert len(tiles) > 1
    rq, rk, rv, _, _ = oracle.attn_bwd(f64(qc), f64(kc), f64(vc), f64(doc), scale)
    for tile in tiles:
        say(f"attn_bwd_tile {tile} bh={bh} n={n} d={d} qx{q_mult}")
        got = at.attn_bwd_tile(tile, q, k, v, o, do, lse, scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"{tile}: {name} differs from the default"
    check(f64(ref[0]), rq, TOL["bf16"], f"dQ {bh}x{n}x{d}", grad_scaled=q_mult > 1.0)
    check(f64(ref[1]), rk, TOL["bf16"], f"dK {bh}x{n}x{d}", grad_scaled=q_mult > 1.0)
    check(f64(ref[2]), rv, TOL["bf16"], f"dV {bh}x{n}x{d}", grad_scaled=q_mult > 1.0)
