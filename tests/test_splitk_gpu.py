"""Parity of the key-split rectangular forward (attn_fwd_splitk) with the
float64 oracle.

Small ragged shapes (one query, fewer queries than keys, more queries than
keys, chunk counts that do and do not divide the key count, one-key tails)
are compared over every element of O and lse.  The two rectangular
workloads are checked at full size: the decoding case over every output (the
oracle needs only one row per head), the 1024-query chunk on rows from every (head, query block).
The merge of chunk partials is stressed with peaked weights (Q x 20), where
the chunks' log-sum-exps differ by hundreds.  Tolerance: max-abs 2e-2 (bf16
inputs, fp32 accumulation).
"""
import pytest
import torch

import aware_tiling_amd as at
import oracle
from aware_tiling_amd.inputs import WORKLOADS, make_inputs
from tests.gpu_util import (TOL, check, f64, gather_rows, oracle_fwd_head_rows, rows_every_block,
                            say)

pytestmark = pytest.mark.gpu

CASES = [
    # (bh, nq, nk, d, splits, seed, q_mult)
    (2, 1, 1000, 128, 0, 201, 1.0),
    (2, 1, 1000, 128, 1, 202, 1.0),
    (2, 1, 1000, 128, 3, 203, 1.0),
    (3, 37, 777, 64, 5, 204, 1.0),
    (1, 300, 129, 128, 2, 205, 1.0),  # more queries than keys, 1-key last chunk
    (2, 130, 4100, 64, 0, 206, 1.0),  # eight-wave kernel (nq > 128)
    (1, 1, 1, 128, 4, 207, 1.0),      # one key
    (1, 5, 65, 64, 2, 208, 1.0),      # chunks of 64 and 1 keys
    (2, 5, 3000, 128, 9, 209, 20.0),  # peaked weights: chunk lse far apart
    (4, 129, 2048, 128, 16, 210, 1.0),
    (2, 3, 1500, 256, 0, 214, 1.0),   # d = 256: four-wave kernel, 32-key steps
    (1, 140, 333, 256, 3, 215, 4.0),  # d = 256, nq > 128, ragged chunks
    (1, 40, 2000, 256, 5, 216, 20.0),  # d = 256, peaked weights
    (3, 20, 1500, 64, 3, 217, 20.0),   # one-wave decoding form, peaked weights
]


def _inputs(bh, nq, nk, d, seed, q_mult):
    qc, kc, vc = make_inputs(bh, nq, d, "bf16", seed, q_mult, nk=nk)
    return (qc, kc, vc), tuple(t.to("cuda") for t in (qc, kc, vc))


@pytest.mark.parametrize("bh,nq,nk,d,splits,seed,q_mult", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-s{c[4]}-q{c[6]:g}" for c in CASES])
def test_splitk_matches_oracle(bh, nq, nk, d, splits, seed, q_mult):
    used = at.splitk_splits(bh, nq, nk, d, splits)
    say(f"attn_fwd_splitk bh={bh} nq={nq} nk={nk} d={d} splits={splits} (uses {used})")
    (qc, kc, vc), (q, k, v) = _inputs(bh, nq, nk, d, seed, q_mult)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd_splitk(q, k, v, splits, scale)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.attn_fwd(f64(qc), f64(kc), f64(vc), scale)
    check(f64(o), ro, TOL["bf16"], f"O {bh}x{nq}x{nk}x{d}/{splits}")
    check(f64(lse), rl, TOL["bf16"], f"lse {bh}x{nq}x{nk}x{d}/{splits}")


def test_splitk_square_agrees_with_fused():
    """nq == nk: with one chunk the key-split call runs the fused schedule
    and matches attn_fwd bit for bit; with three chunks each chunk rounds its
    weights to bf16 against its own running maximum, so it agrees with the
    oracle to the same bar as attn_fwd does (not bit for bit)."""
    (qc, kc, vc), (q, k, v) = _inputs(2, 500, 500, 128, 211, 1.0)
    o1, l1 = at.attn_fwd(q, k, v)
    o2, l2 = at.attn_fwd_splitk(q, k, v, 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = at.attn_fwd_splitk(q, k, v, 3)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.attn_fwd(f64(qc), f64(kc), f64(vc), at.default_scale(128))
    check(f64(o3), ro, TOL["bf16"], "split 3 O")
    check(f64(l3), rl, TOL["bf16"], "split 3 lse")


def test_splitk_decode_workload_every_output():
    w = WORKLOADS["decode_bf16_b8h32_q1_k16384_d128"]
    say(f"attn_fwd_splitk full workload {w.name}")
    qc, kc, vc = make_inputs(w.bh, w.queries, w.d, w.dtype, w.seed, w.q_mult, nk=w.n)
    q, k, v = (t.to("cuda") for t in (qc, kc, vc))
    o, lse = at.attn_fwd_splitk(q, k, v, 0, w.scale)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.attn_fwd(f64(qc), f64(kc), f64(vc), w.scale)
    check(f64(o), ro, TOL["bf16"], "O decode (all heads)")
    check(f64(lse), rl, TOL["bf16"], "lse decode (all heads)")
    # repeated calls are bitwise identical
    o2, lse2 = at.attn_fwd_splitk(q, k, v, 0, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_splitk_chunk_workload_sampled_rows():
    w = WORKLOADS["chunk_bf16_b1h32_q1024_k16384_d128"]
    say(f"attn_fwd_splitk full workload {w.name}")
    qc, kc, vc = make_inputs(w.bh, w.queries, w.d, w.dtype, w.seed, w.q_mult, nk=w.n)
    q, k, v = (t.to("cuda") for t in (qc, kc, vc))
    o, lse = at.attn_fwd_splitk(q, k, v, 0, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # rows from every (head, 256-query block) of the eight-wave split kernel
    rows = rows_every_block(w.bh, w.queries, 256, 2, w.seed)
    ro, rl = oracle_fwd_head_rows(qc, kc, vc, w.scale, rows)
    check(gather_rows(o, rows), ro, TOL["bf16"], "O chunk every block")
    check(gather_rows(lse, rows), rl, TOL["bf16"], "lse chunk every block")


def test_splitk_rejects_bad_arguments():
    (_, (q, k, v)) = _inputs(1, 4, 100, 128, 212, 1.0)
    with pytest.raises(at.AttnError):
        at.attn_fwd_splitk(q, k, v, 300)
    (_, (q2, k2, v2)) = _inputs(1, 4, 100, 96, 213, 1.0)
    with pytest.raises(at.AttnError):
        at.attn_fwd_splitk(q2, k2, v2, 2)
    # no keys: undefined softmax, refused
    with pytest.raises(at.AttnError):
        at.attn_fwd_splitk(q, k[:, :0].contiguous(), v[:, :0].contiguous(), 1)
