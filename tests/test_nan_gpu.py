"""NaN inputs propagate to exactly the outputs that depend on them.

No entry point inspects its inputs.  A NaN in query row i makes O row i and
lse i NaN (every score of that row is NaN); a NaN in key row j makes every
row of that head NaN (every query weighs key j); a NaN in V[j][c] makes
column c of every row of that head NaN and leaves the other columns and lse
as they were.  Rows, columns and heads the NaN does not reach must still
match the float64 oracle on the clean inputs (max-abs 2e-2, bf16 inputs).
Covered: attn_fwd (d 64, 128, 256), attn_fwd_smallcache and attn_fwd_budget
(d 256).
"""
import numpy as np
import pytest
import torch

import aware_tiling_amd as at
from tests.gpu_util import TOL, check, f64, inputs, oracle_fwd_rows, say

pytestmark = pytest.mark.gpu

BH, N = 2, 200


def _paths(d):
    s = at.default_scale(d)
    paths = [("attn_fwd", lambda q, k, v: at.attn_fwd(q, k, v, s))]
    if d == 256:
        paths.append(("attn_fwd_smallcache",
                      lambda q, k, v: at.attn_fwd_smallcache(q, k, v, 49152, s)))
        paths.append(("attn_fwd_budget",
                      lambda q, k, v: at.attn_fwd_budget(q, k, v, at.fwd_budget_onchip_elems(d),
                                                         s)))
    return s, paths


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("where", ["q_row", "k_row", "v_elem"])
def test_nan_reaches_only_its_dependents(d, where):
    seed = 900 + d + {"q_row": 0, "k_row": 1, "v_elem": 2}[where]
    (qc, kc, vc), (q, k, v) = inputs(BH, N, d, "bf16", seed)
    scale, paths = _paths(d)
    ro, rl = oracle_fwd_rows(qc, kc, vc, scale, np.arange(BH), np.arange(N))
    i, j, col = 37, 123, 5  # poisoned query row, key row, value column (head 1)
    q, k, v = q.clone(), k.clone(), v.clone()
    if where == "q_row":
        q[1, i, 3] = float("nan")
    elif where == "k_row":
        k[1, j, 3] = float("nan")
    else:
        v[1, j, col] = float("nan")
    for name, fn in paths:
        say(f"{name} d={d} NaN in {where}")
        o, lse = fn(q, k, v)
        torch.cuda.synchronize()
        o, lse = f64(o), f64(lse)
        # head 0 never sees the NaN
        check(o[0], ro[0], TOL["bf16"], f"{name} O head 0")
        check(lse[0], rl[0], TOL["bf16"], f"{name} lse head 0")
        if where == "q_row":
            assert np.isnan(o[1, i]).all() and np.isnan(lse[1, i])
            keep = np.arange(N) != i
            check(o[1, keep], ro[1, keep], TOL["bf16"], f"{name} O other rows")
            check(lse[1, keep], rl[1, keep], TOL["bf16"], f"{name} lse other rows")
        elif where == "k_row":
            assert np.isnan(o[1]).all() and np.isnan(lse[1]).all()
        else:
            assert np.isnan(o[1, :, col]).all()
            keep = np.arange(d) != col
            check(o[1][:, keep], ro[1][:, keep], TOL["bf16"], f"{name} O other columns")
            check(lse[1], rl[1], TOL["bf16"], f"{name} lse")
