"""Parity of the fused streaming forward (attn_fwd) with the float64 oracle.

Small shapes are compared element by element over all of O and lse; they
span several query blocks and key tiles and end in ragged tails.  The
full-size workloads are compared on rows drawn from every (head, query
block), so every workgroup of the launch is checked (the oracle computes
those rows one by one over all keys), and, over every element, against the
convex-hull property that holds at any size (each output row is a weighted
average of value rows, so it lies between their column minima and maxima).
Tolerances: max-abs 1e-5 for fp32 inputs, 2e-2 for bf16 inputs.
"""

import numpy as np
import pytest
import torch

import aware_tiling_amd as at
from aware_tiling_amd.inputs import TORCH_DTYPES, WORKLOADS
from tests.gpu_util import (TOL, check, f64, gather_rows, inputs, oracle_fwd_head_rows,
                            oracle_fwd_rows, rows_every_block, say)

pytestmark = pytest.mark.gpu

SMALL = [
    # (bh, n, d, dtype, seed, q_mult)
    (1, 256, 64, "f32", 1, 1.0),  # the tiny fp32 workload, compared in full
    (2, 300, 64, "f32", 11, 1.0),
    (1, 129, 128, "f32", 12, 1.0),
    (1, 1, 64, "f32", 13, 1.0),
    (1, 200, 256, "f32", 14, 1.0),
    (2, 65, 256, "f32", 15, 4.0),
    (2, 300, 64, "bf16", 21, 1.0),
    (3, 1000, 128, "bf16", 22, 1.0),
    (1, 257, 256, "bf16", 23, 1.0),
    (1, 1, 128, "bf16", 24, 1.0),
    (2, 17, 64, "bf16", 25, 1.0),
    (1, 255, 128, "bf16", 26, 1.0),
    (2, 96, 256, "bf16", 27, 1.0),
    (2, 513, 128, "bf16", 28, 4.0),
    (1, 700, 64, "bf16", 29, 40.0),  # scores in the hundreds: max-rescaling path
    (1, 640, 128, "bf16", 30, 40.0),
    (1, 500, 256, "bf16", 31, 40.0),  # d = 256: maximum taken only when a tile sum shows it moved
]


def _run_full(bh, n, d, dtype, seed, q_mult):
    (qc, kc, vc), (q, k, v) = inputs(bh, n, d, dtype, seed, q_mult)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    ro, rl = oracle_fwd_rows(qc, kc, vc, scale, np.arange(bh), np.arange(n))
    tol = TOL[dtype]
    check(f64(o), ro, tol, f"O {bh}x{n}x{d} {dtype} qx{q_mult}")
    check(f64(lse), rl, tol, f"lse {bh}x{n}x{d} {dtype}")


@pytest.mark.parametrize("bh,n,d,dtype,seed,q_mult", SMALL,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-q{c[5]:g}" for c in SMALL])
def test_fwd_matches_oracle_small(bh, n, d, dtype, seed, q_mult):
    say(f"attn_fwd small case bh={bh} n={n} d={d} {dtype} seed={seed} qx{q_mult}")
    _run_full(bh, n, d, dtype, seed, q_mult)


# Every compiled tile shape of the bf16 kernel (the default and the d = 128
# sweep shapes), on ragged shapes, through the explicitly named entry point.
TILES = {64: ["g2x64p"],
         128: ["d8x64", "r64c32", "r64c64", "r128c32", "r128c64", "r256c32", "r256c64"],
         256: ["d4x32b"]}


@pytest.mark.parametrize("d,tile", [(d, t) for d, ts in TILES.items() for t in ts])
def test_fwd_every_tile_shape(d, tile):
    say(f"attn_fwd_tile {tile} d={d}")
    (qc, kc, vc), (q, k, v) = inputs(2, 333, d, "bf16", 40 + d, 2.0)
    scale = at.default_scale(d)
    o, lse = at.attn_fwd_tile(tile, q, k, v, scale)
    torch.cuda.synchronize()
    ro, rl = oracle_fwd_rows(qc, kc, vc, scale, np.arange(2), np.arange(333))
    check(f64(o), ro, TOL["bf16"], f"O tile {tile}")
    check(f64(lse), rl, TOL["bf16"], f"lse tile {tile}")


def _full_workload(name, per_block=2):
    w = WORKLOADS[name]
    say(f"attn_fwd full workload {name}")
    (qc, kc, vc), (q, k, v) = inputs(w.bh, w.n, w.d, w.dtype, w.seed, w.q_mult)
    o, lse = at.attn_fwd(q, k, v, w.scale)
    torch.cuda.synchronize()
    # property over every element: rows of O lie in the columnwise hull of V
    vf = v.float()
    lo = vf.amin(dim=1, keepdim=True)
    hi = vf.amax(dim=1, keepdim=True)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    slack = 1e-3
    assert bool(((o >= lo - slack) & (o <= hi + slack)).all()), "O outside the hull of V"
    # rows from every (head, query block), i.e. from every workgroup of the
    # launch, against the oracle
    block = at.fwd_query_block(w.d, TORCH_DTYPES[w.dtype])
    rows = rows_every_block(w.bh, w.n, block, per_block, w.seed)
    say(f"  oracle on {rows.size} rows: {per_block} from each of {w.bh} heads x "
        f"{-(-w.n // block)} query blocks of {block}")
    ro, rl = oracle_fwd_head_rows(qc, kc, vc, w.scale, rows)
    check(gather_rows(o, rows), ro, TOL[w.dtype], f"O every block {name}")
    check(gather_rows(lse, rows), rl, TOL[w.dtype], f"lse every block {name}")
    return o, lse, (q, k, v)


def test_fwd_full_f32_workload():
    _full_workload("fwd_f32_h1_n256_d64", 64)


def test_fwd_full_teaching_shape():
    _full_workload("fwd_bf16_b4h16_n4096_d64")


def test_fwd_full_long_sequence_large_scores():
    o, lse, (q, k, v) = _full_workload("fwd_bf16_b1h32_n16384_d128_qx4")
    # bitwise determinism at full size
    o2, lse2 = at.attn_fwd(q, k, v, WORKLOADS["fwd_bf16_b1h32_n16384_d128_qx4"].scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_fwd_d256_fused_on_small_cache_shape():
    _full_workload("smallcache_bf16_b1h8_n4096_d256")


def test_fwd_deterministic_repeat():
    (_, (q, k, v)) = inputs(3, 777, 128, "bf16", 50, 1.0)
    outs = [at.attn_fwd(q, k, v) for _ in range(5)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_fwd_without_lse_and_into_given_output():
    (qc, kc, vc), (q, k, v) = inputs(1, 200, 64, "bf16", 51)
    out = torch.full((1, 200, 64), float("nan"), device="cuda")
    o, lse = at.attn_fwd(q, k, v, out=out, lse=False)
    torch.cuda.synchronize()
    assert lse is None and o.data_ptr() == out.data_ptr()
    ro, _ = oracle_fwd_rows(qc, kc, vc, at.default_scale(64), np.arange(1), np.arange(200))
    check(f64(o), ro, TOL["bf16"], "O into given buffer")


def test_fwd_empty_is_noop():
    q = torch.empty((0, 128, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = at.attn_fwd(q, q, q)
    assert o.shape == (0, 128, 64)
    q = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = at.attn_fwd(q, q, q)
    assert o.shape == (2, 0, 64)


def test_fwd_rejects_bad_arguments_on_gpu():
    q = torch.zeros((1, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(at.AttnError):
        at.attn_fwd(q, q, q)
    q = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(at.AttnError):
        at.attn_fwd(q, q, q, scale=-1.0)
