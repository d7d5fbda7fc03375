"""Helpers for GPU parity tests: seeded inputs, oracle on sampled rows, and
error reporting.  The oracle always sees exactly the values the GPU sees
(bf16/fp32 widened to float64)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from aware_tiling_amd.inputs import make_inputs

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """First and last rows of the sequence plus seeded random rows."""
    edge = min(count // 4, n)
    rows = set(range(edge)) | set(range(max(0, n - edge), n))
    rng = np.random.default_rng(seed)
    rows |= set(rng.choice(n, size=min(n, count - len(rows)), replace=False).tolist())
    return np.array(sorted(rows)[:max(count, 1)])


def oracle_fwd_rows(q, k, v, scale, heads, rows):
    """Oracle O and lse for the given heads and query rows (all keys)."""
    qs = f64(q[heads][:, rows])
    o, lse, _ = oracle.attn_fwd(qs, f64(k[heads]), f64(v[heads]), scale)
    return o, lse


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / den if den > 0 else float(np.linalg.norm(a - b))


def check(got: np.ndarray, ref: np.ndarray, tol: float, what: str, grad_scaled: bool = False):
    """Max-abs comparison against the absolute bar ``tol``.

    ``grad_scaled`` is for gradients of stress inputs whose queries were
    multiplied beyond the stated workloads: gradients grow with that factor
    (dQ, dK carry the scores' slope), so there the bar is tol times
    max(1, max|ref|).  Forward outputs never take it: O is a convex
    combination of value rows and lse an exponent, so their error does not
    grow with the scores and the absolute bar holds for every input."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = max_abs(got, ref)
    big = float(np.max(np.abs(ref))) if ref.size else 0.0
    lim = tol * max(1.0, big) if grad_scaled else tol
    say(f"  {what}: max|err| {err:.3e} (bar {lim:.3g}), max|ref| {big:.3g}, "
        f"rel fro {rel_fro(got, ref):.2e}")
    assert err <= lim, f"{what}: max abs error {err:.3e} > {lim:.3g}"


def rows_every_block(bh: int, n: int, block: int, per_block: int, seed: int) -> np.ndarray:
    """Query rows [bh, nb * per_block] that reach every (head, query block)
    of ``block`` rows: per head and block, ``per_block`` seeded rows inside
    the block (distinct where the block is long enough; a short ragged last
    block repeats its rows), with the sequence's first and last rows always
    included.  Rows differ from head to head, so each workgroup is sampled
    at varied lane offsets."""
    rng = np.random.default_rng(seed)
    nb = -(-n // block)
    out = np.empty((bh, nb * per_block), dtype=np.int64)
    for h in range(bh):
        rows = []
        for b in range(nb):
            lo, hi = b * block, min(n, (b + 1) * block)
            size = hi - lo
            pick = lo + rng.choice(size, size=per_block, replace=size < per_block)
            if b == 0:
                pick[0] = 0
            if b == nb - 1:
                pick[-1] = n - 1
            rows.extend(pick.tolist())
        out[h] = rows
    return out


def oracle_fwd_head_rows(q, k, v, scale, rows):
    """Oracle O and lse for per-head query rows ``rows`` [bh, r] (all keys of
    each head)."""
    idx = torch.as_tensor(rows)
    qs = torch.stack([q[h, idx[h]] for h in range(q.shape[0])])
    o, lse, _ = oracle.attn_fwd(f64(qs), f64(k), f64(v), scale)
    return o, lse


def gather_rows(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """t[h, rows[h]] for every head, as float64 (t is [bh, n, ...])."""
    idx = torch.as_tensor(rows, device=t.device)
    return np.stack([f64(t[h, idx[h]]) for h in range(t.shape[0])])


def inputs(bh, n, d, dtype, seed, q_mult=1.0, with_do=False, device="cuda"):
    ts = make_inputs(bh, n, d, dtype, seed, q_mult, with_do=with_do)
    return ts, tuple(t.to(device) for t in ts)
