"""Parity of the block-sparse forward (attn_fwd_blocksparse) with the
float64 oracle's block-masked definition.

Masks keep 128 x 128 blocks.  Small ragged shapes (per-head and shared
masks, a partial last block, query blocks with no kept key, a mask that keeps
only the partial last key block, all blocks kept) are compared over every
element; the block-sparse workload (batch 1 x 32 heads, N 16384, d 128, a
quarter of the blocks kept) on rows from every (head, query block).  Rows with no
kept key must give O = 0 and lse = -inf exactly.  Tolerance: max-abs 2e-2
(bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import aware_tiling_amd as at
import oracle
from aware_tiling_amd.inputs import WORKLOADS, make_block_mask, workload_inputs
from tests.gpu_util import TOL, check, f64, gather_rows, inputs, rows_every_block, say

pytestmark = pytest.mark.gpu

B = at.SPARSE_BLOCK


def _run(bh, n, d, seed, q_mult, mask):
    (qc, kc, vc), (q, k, v) = inputs(bh, n, d, "bf16", seed, q_mult)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd_blocksparse(q, k, v, mask.to("cuda"), scale)
    torch.cuda.synchronize()
    return (qc, kc, vc), (o, lse), scale


def _compare(qc, kc, vc, o, lse, scale, mask, what):
    ro, rl, _ = oracle.attn_fwd_masked(f64(qc), f64(kc), f64(vc), scale, mask.numpy(), B, B)
    go, gl = f64(o), f64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), f"{what}: rows with no kept key differ"
    assert np.all(go[empty] == 0.0), f"{what}: O of rows with no kept key is not 0"
    check(go[~empty], ro[~empty], TOL["bf16"], f"O {what}")
    check(gl[~empty], rl[~empty], TOL["bf16"], f"lse {what}")


CASES = [
    # (bh, n, d, seed, q_mult, mask_heads, density, keep_diagonal)
    (2, 300, 128, 401, 1.0, 2, 0.5, True),
    (1, 1000, 64, 402, 1.0, 1, 0.3, True),
    (3, 129, 128, 403, 1.0, 3, 0.4, False),   # may leave query blocks empty
    (2, 640, 64, 404, 1.0, 2, 0.35, False),
    (1, 257, 128, 405, 1.0, 1, 1.0, True),     # every block kept
    (1, 700, 128, 406, 20.0, 1, 0.5, True),    # peaked weights
    (2, 333, 256, 407, 1.0, 1, 0.5, False),    # d = 256, last 64-key tile < 32 keys
    (1, 300, 256, 408, 4.0, 1, 1.0, True),     # last 32 keys partial
    (1, 500, 256, 409, 20.0, 1, 0.5, True),    # d = 256, peaked weights
]


@pytest.mark.parametrize("bh,n,d,seed,q_mult,mh,density,diag", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-m{c[5]}-p{c[6]:g}" for c in CASES])
def test_blocksparse_matches_oracle(bh, n, d, seed, q_mult, mh, density, diag):
    nb = -(-n // B)
    mask = make_block_mask(mh, nb, density, seed + 1000, keep_diagonal=diag)
    say(f"attn_fwd_blocksparse bh={bh} n={n} d={d} mask_heads={mh} kept {int(mask.sum())}/"
        f"{mask.numel()} blocks")
    (qc, kc, vc), (o, lse), scale = _run(bh, n, d, seed, q_mult, mask)
    _compare(qc, kc, vc, o, lse, scale, mask, f"{bh}x{n}x{d}")


def test_blocksparse_edge_masks():
    bh, n, d = 2, 300, 128  # 3 blocks, the last one 44 keys
    nb = 3
    mask = torch.zeros((bh, nb, nb), dtype=torch.uint8)
    mask[0, 0, 2] = 1          # head 0, query block 0: only the partial last key block
    mask[0, 2, 1] = 1          # head 0, query block 2 (partial): one full key block
    mask[1, 1, :] = 1          # head 1, query block 1: everything; blocks 0, 2 empty
    say("attn_fwd_blocksparse edge masks")
    (qc, kc, vc), (o, lse), scale = _run(bh, n, d, 407, 1.0, mask)
    _compare(qc, kc, vc, o, lse, scale, mask, "edge masks")
    # all-empty mask: every row O = 0, lse = -inf
    (_, (o0, l0), _) = _run(1, 200, 64, 408, 1.0, torch.zeros((1, 2, 2), dtype=torch.uint8))
    assert torch.all(o0 == 0) and torch.all(torch.isneginf(l0))


def test_blocksparse_all_kept_matches_fused():
    (qc, kc, vc), (q, k, v) = inputs(2, 500, 128, "bf16", 409)
    mask = torch.ones((1, 4, 4), dtype=torch.uint8, device="cuda")
    o1, l1 = at.attn_fwd(q, k, v)
    o2, l2 = at.attn_fwd_blocksparse(q, k, v, mask)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.attn_fwd(f64(qc), f64(kc), f64(vc), at.default_scale(128))
    check(f64(o2), ro, TOL["bf16"], "all kept O vs oracle")
    check(f64(l2), rl, TOL["bf16"], "all kept lse vs oracle")
    check(f64(o2), f64(o1), TOL["bf16"], "all kept O vs attn_fwd")


def test_blocksparse_workload_sampled_rows():
    w = WORKLOADS["sparse_bf16_b1h32_n16384_d128_keep25"]
    nb = -(-w.n // B)
    mask = make_block_mask(w.bh, nb, w.density, w.seed + 1000)
    say(f"attn_fwd_blocksparse full workload {w.name}: kept {float(mask.float().mean()):.3f}")
    qc, kc, vc = workload_inputs(w)
    q, k, v = (t.to("cuda") for t in (qc, kc, vc))
    o, lse = at.attn_fwd_blocksparse(q, k, v, mask.to("cuda"), w.scale)
    o2, lse2 = at.attn_fwd_blocksparse(q, k, v, mask.to("cuda"), w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # rows from every (head, 128-query block): every workgroup of the launch
    rows = rows_every_block(w.bh, w.n, B, 2, w.seed)
    idx = torch.as_tensor(rows)
    qs = torch.stack([qc[h, idx[h]] for h in range(w.bh)])
    row_mask = np.stack([mask[h, rows[h] // B, :].numpy() for h in range(w.bh)])
    say(f"  masked oracle on {rows.size} rows (one query per mask row)")
    ro, rl, _ = oracle.attn_fwd_masked(f64(qs), f64(kc), f64(vc), w.scale, row_mask, 1, B)
    check(gather_rows(o, rows), ro, TOL["bf16"], "O sparse every block")
    check(gather_rows(lse, rows), rl, TOL["bf16"], "lse sparse every block")


def test_blocksparse_rejects_bad_arguments():
    (_, (q, k, v)) = inputs(1, 200, 128, "bf16", 410)
    with pytest.raises(ValueError):
        at.attn_fwd_blocksparse(q, k, v, torch.ones((1, 3, 3), dtype=torch.uint8, device="cuda"))
    (_, (q2, k2, v2)) = inputs(1, 200, 96, "bf16", 411)
    with pytest.raises(at.AttnError):
        at.attn_fwd_blocksparse(q2, k2, v2, torch.ones((1, 2, 2), dtype=torch.uint8,
                                                       device="cuda"))
