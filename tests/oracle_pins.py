"""Pins for the float64 oracle: checks against facts the pages and the
mathematics fix, independent of the oracle's own code.

Each pin is a function ``pin(lib)`` that raises AssertionError on failure, so
the same battery runs against the real oracle (tests/test_oracle.py) and
against deliberately broken copies of it (tests/test_oracle_mutants.py, which
shows that a plausible slip in the oracle is caught by at least one pin).

Definition pinned (page 1, "Attention as a mathematical problem"):
s_ij = scale <q_i, k_j>, p_ij = softmax_j(s_ij), o_i = sum_j p_ij v_j.
Streaming recurrence pinned (page 1, "Softmax without storing the score
matrix").  Square-tile schedule pinned (page 1, "Small caches").  The
block-masked definition (page 3's sparse attention) pinned against plain
attention over each row's kept keys.  Gradients pinned by finite
differences of the forward and by closed forms.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_forms.json")


def _ev(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log}))  # noqa: S307


def _arr(rows):
    if isinstance(rows[0], list):
        return np.array([[_ev(x) for x in r] for r in rows])
    return np.array([_ev(x) for x in rows])


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(seed, bh, nq, nk, d, qs=1.0):
    r = _rng(seed)
    return (r.standard_normal((bh, nq, d)) * qs, r.standard_normal((bh, nk, d)),
            r.standard_normal((bh, nk, d)))


def _close(a, b, atol, rtol=0.0, what=""):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e} (atol {atol}, rtol {rtol})"


def _torch_fwd(q, k, v, scale):
    """Library routine path: torch float64 softmax and matmul."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2))
    return (torch.matmul(torch.softmax(s, dim=-1), tv).numpy(),
            torch.logsumexp(s, dim=-1).numpy())


# --------------------------------------------------------------------------
# forward pins


def pin_golden_forward(lib):
    for c in json.load(open(GOLDEN))["forward"]:
        q, k, v = (_arr(c[x])[None] for x in ("Q", "K", "V"))
        o, lse, _ = oracle.attn_fwd(q, k, v, _ev(c["scale"]), lib=lib)
        _close(o[0], _arr(c["O"]), 1e-13, 1e-13, c["name"] + " O")
        _close(lse[0], _arr(c["lse"]), 1e-13, 1e-13, c["name"] + " lse")


def pin_torch_library(lib):
    shapes = [(1, 1, 1, 1), (2, 17, 17, 5), (3, 64, 33, 16), (1, 40, 512, 64), (2, 9, 3, 7),
              (3, 1, 700, 8)]
    for i, (bh, nq, nk, d) in enumerate(shapes):
        q, k, v = _rand(100 + i, bh, nq, nk, d)
        scale = 1.0 / math.sqrt(d)
        o, lse, _ = oracle.attn_fwd(q, k, v, scale, lib=lib)
        ro, rl = _torch_fwd(q, k, v, scale)
        _close(o, ro, 1e-12, 1e-12, f"torch O {bh,nq,nk,d}")
        _close(lse, rl, 1e-12, 1e-12, f"torch lse {bh,nq,nk,d}")


def pin_identity_values_give_weights(lib):
    """With V = I (d = N keys), row i of O is the weight row p_i: it must sum
    to one and equal exp(s_ij) / sum_t exp(s_it) computed without any shift."""
    n = 12
    q, k, _ = _rand(7, 1, 5, n, n)
    v = np.eye(n)[None]
    scale = 0.3
    o, _, _ = oracle.attn_fwd(q, k, v, scale, lib=lib)
    s = scale * q[0] @ k[0].T
    brute = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    _close(o[0], brute, 1e-14, 1e-13, "weights")
    _close(o[0].sum(axis=1), np.ones(5), 1e-14, 0, "row sums")


def pin_constant_values(lib):
    q, k, _ = _rand(8, 2, 9, 31, 6)
    c = np.array([1.5, -2.0, 0.0, 3.25, 7.0, -0.125])
    v = np.broadcast_to(c, (2, 31, 6)).copy()
    o, _, _ = oracle.attn_fwd(q, k, v, 0.7, lib=lib)
    _close(o, np.broadcast_to(c, o.shape), 1e-14, 1e-14, "constant V")


def pin_zero_queries_mean_pool(lib):
    _, k, v = _rand(9, 2, 4, 23, 5)
    q = np.zeros((2, 4, 5))
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.5, lib=lib)
    _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), 1e-14, 1e-13,
           "mean pooling")
    _close(lse, np.full((2, 4), math.log(23)), 1e-14, 1e-14, "lse log N")


def pin_single_key(lib):
    q, k, v = _rand(10, 3, 6, 1, 4)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.9, lib=lib)
    _close(o, np.broadcast_to(v, o.shape), 0, 0, "N=1 gives V")
    _close(lse, 0.9 * np.einsum("bqd,bkd->bq", q, k), 1e-14, 1e-14, "N=1 lse")


def pin_two_keys_logistic(lib):
    q, k, v = _rand(11, 1, 7, 2, 3)
    scale = 1.3
    o, _, _ = oracle.attn_fwd(q, k, v, scale, lib=lib)
    s = scale * q[0] @ k[0].T
    p1 = 1.0 / (1.0 + np.exp(-(s[:, 0] - s[:, 1])))
    ref = p1[:, None] * v[0, 0] + (1 - p1)[:, None] * v[0, 1]
    _close(o[0], ref, 1e-14, 1e-13, "logistic")


def pin_permutations(lib):
    q, k, v = _rand(12, 2, 13, 29, 8)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.4, lib=lib)
    pk = _rng(1).permutation(29)
    o2, lse2, _ = oracle.attn_fwd(q, k[:, pk], v[:, pk], 0.4, lib=lib)
    _close(o2, o, 1e-14, 1e-13, "key permutation")
    _close(lse2, lse, 1e-14, 1e-13, "key permutation lse")
    pq = _rng(2).permutation(13)
    o3, lse3, _ = oracle.attn_fwd(q[:, pq], k, v, 0.4, lib=lib)
    _close(o3, o[:, pq], 0, 0, "query permutation")
    _close(lse3, lse[:, pq], 0, 0, "query permutation lse")


def pin_shift_and_linearity(lib):
    q, k, v = _rand(13, 1, 10, 21, 6)
    scale = 0.6
    o, lse, _ = oracle.attn_fwd(q, k, v, scale, lib=lib)
    c = _rng(3).standard_normal(6)
    o2, lse2, _ = oracle.attn_fwd(q, k + c, v, scale, lib=lib)
    _close(o2, o, 1e-13, 1e-12, "key shift")
    _close(lse2, lse + scale * (q @ c), 1e-12, 1e-12, "key shift lse")
    o3, _, _ = oracle.attn_fwd(q, k, v + c, scale, lib=lib)
    _close(o3, o + c, 1e-13, 1e-12, "value shift")
    _, _, w = _rand(14, 1, 10, 21, 6)
    ow, _, _ = oracle.attn_fwd(q, k, w, scale, lib=lib)
    ol, _, _ = oracle.attn_fwd(q, k, 2.0 * v - 3.0 * w, scale, lib=lib)
    _close(ol, 2.0 * o - 3.0 * ow, 1e-12, 1e-12, "linear in V")


def pin_large_scores(lib):
    """Scores far beyond exp's double range stay finite; with a clear winner
    the output is that key's value (the softmax argmax limit)."""
    r = _rng(15)
    n, d = 16, 4
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    q = 400.0 * k[:, [3, 11, 0, 7]]  # large queries, scores in the hundreds
    s = q[0] @ k[0].T
    assert np.abs(s).max() > 800.0  # exp overflows without the shift
    top = np.sort(s, axis=1)
    assert np.all(top[:, -1] - top[:, -2] > 60.0)
    win = np.argmax(s, axis=1)
    o, lse, _ = oracle.attn_fwd(q, k, v, 1.0, lib=lib)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    _close(o[0], v[0, win], 1e-12, 1e-12, "argmax limit")
    _close(lse[0], s.max(axis=1), 1e-12, 1e-12, "lse at the limit")


def pin_large_scores_stream_and_square(lib):
    """The running maximum and the per-tile maxima are what keep the
    exponentials finite: with scores spanning thousands, the streaming and
    square-tile schedules still agree with the direct definition."""
    r = _rng(26)
    n, d = 24, 4
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    q = 300.0 * r.standard_normal((1, 6, d))
    s = q[0] @ k[0].T
    assert np.ptp(s, axis=1).min() > 1000.0
    o, lse, _ = oracle.attn_fwd(q, k, v, 1.0, lib=lib)
    for blk in (1, 3, 5, 16):
        o2, lse2, _ = oracle.attn_fwd_stream(q, k, v, 1.0, blk, lib=lib)
        _close(o2, o, 1e-12, 1e-12, f"large stream {blk}")
        _close(lse2, lse, 1e-12, 1e-12, f"large stream lse {blk}")
        o3, lse3, _ = oracle.attn_fwd_square(q, k, v, 1.0, blk, lib=lib)
        _close(o3, o, 1e-12, 1e-12, f"large square {blk}")
        _close(lse3, lse, 1e-12, 1e-12, f"large square lse {blk}")


def pin_streaming_equals_direct(lib):
    q, k, v = _rand(16, 2, 11, 70, 9, qs=3.0)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.8, lib=lib)
    for blk in (1, 7, 64, 70, 200):
        o2, lse2, _ = oracle.attn_fwd_stream(q, k, v, 0.8, blk, lib=lib)
        _close(o2, o, 1e-12, 1e-12, f"stream block {blk}")
        _close(lse2, lse, 1e-12, 1e-12, f"stream lse block {blk}")


def pin_square_equals_direct(lib):
    q, k, v = _rand(17, 2, 11, 70, 9, qs=3.0)
    o, lse, _ = oracle.attn_fwd(q, k, v, 0.8, lib=lib)
    for b in (1, 5, 32, 70, 128):
        o2, lse2, _ = oracle.attn_fwd_square(q, k, v, 0.8, b, lib=lib)
        _close(o2, o, 1e-12, 1e-12, f"square b {b}")
        _close(lse2, lse, 1e-12, 1e-12, f"square lse b {b}")


def pin_stream_and_square_vs_torch(lib):
    q, k, v = _rand(18, 1, 6, 37, 5, qs=5.0)
    ro, rl = _torch_fwd(q, k, v, 0.9)
    for blk in (1, 4, 37):
        o, lse, _ = oracle.attn_fwd_stream(q, k, v, 0.9, blk, lib=lib)
        _close(o, ro, 1e-12, 1e-12, f"stream vs torch {blk}")
        _close(lse, rl, 1e-12, 1e-12, f"stream lse vs torch {blk}")
        o, lse, _ = oracle.attn_fwd_square(q, k, v, 0.9, blk, lib=lib)
        _close(o, ro, 1e-12, 1e-12, f"square vs torch {blk}")
        _close(lse, rl, 1e-12, 1e-12, f"square lse vs torch {blk}")


def pin_thread_count(lib):
    q, k, v = _rand(19, 3, 50, 40, 8)
    o1, l1, t1 = oracle.attn_fwd(q, k, v, 0.5, threads=1, lib=lib)
    o8, l8, t8 = oracle.attn_fwd(q, k, v, 0.5, threads=8, lib=lib)
    assert t1 == 1 and t8 == 8
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)


# --------------------------------------------------------------------------
# backward pins


def pin_golden_backward(lib):
    for c in json.load(open(GOLDEN))["backward"]:
        q, k, v, do = (_arr(c[x])[None] for x in ("Q", "K", "V", "dO"))
        dq, dk, dv, D, _ = oracle.attn_bwd(q, k, v, do, _ev(c["scale"]), lib=lib)
        for name, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
            _close(got[0], _arr(c[name]), 1e-13, 1e-13, f"{c['name']} {name}")
        _close(D[0], _arr(c["D"]), 1e-13, 1e-13, f"{c['name']} D")


def _loss(q, k, v, do, scale, lib):
    o, _, _ = oracle.attn_fwd(q, k, v, scale, lib=lib)
    return float(np.sum(o * do))


def pin_finite_differences(lib):
    """Central differences of L = sum(dO * O) through the forward oracle."""
    for seed, (nq, nk, d) in ((20, (3, 5, 2)), (21, (8, 8, 4)), (22, (1, 7, 3))):
        q, k, v = _rand(seed, 1, nq, nk, d, qs=1.5)
        do = _rng(seed + 50).standard_normal((1, nq, d))
        scale = 0.7
        dq, dk, dv, _, _ = oracle.attn_bwd(q, k, v, do, scale, lib=lib)
        h = 1e-6
        for x, g, nm in ((q, dq, "dQ"), (k, dk, "dK"), (v, dv, "dV")):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xp[idx] += h
                lp = _loss(*(xp if y is x else y for y in (q, k, v)), do, scale, lib)
                xp[idx] -= 2 * h
                lm = _loss(*(xp if y is x else y for y in (q, k, v)), do, scale, lib)
                fd[idx] = (lp - lm) / (2 * h)
            _close(g, fd, 1e-7, 1e-6, f"finite differences {nm} seed {seed}")


def pin_autograd(lib):
    for seed, (bh, nq, nk, d) in ((23, (2, 9, 13, 5)), (24, (1, 33, 17, 16))):
        q, k, v = _rand(seed, bh, nq, nk, d, qs=2.0)
        do = _rng(seed + 60).standard_normal((bh, nq, d))
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        s = scale * torch.matmul(tq, tk.transpose(-1, -2))
        o = torch.matmul(torch.softmax(s, dim=-1), tv)
        o.backward(torch.from_numpy(do))
        dq, dk, dv, D, _ = oracle.attn_bwd(q, k, v, do, scale, lib=lib)
        _close(dq, tq.grad.numpy(), 1e-12, 1e-11, "autograd dQ")
        _close(dk, tk.grad.numpy(), 1e-12, 1e-11, "autograd dK")
        _close(dv, tv.grad.numpy(), 1e-12, 1e-11, "autograd dV")
        _close(D, np.sum(do * o.detach().numpy(), axis=-1), 1e-12, 1e-11, "D = <dO, O>")


def pin_gradient_invariants(lib):
    q, k, v = _rand(25, 2, 19, 23, 6, qs=2.0)
    do = _rng(70).standard_normal((2, 19, 6))
    dq, dk, dv, D, _ = oracle.attn_bwd(q, k, v, do, 0.5, lib=lib)
    # a common shift of all keys changes no weight, so sum_j dk_j = 0
    _close(dk.sum(axis=1), np.zeros((2, 6)), 1e-12, 0, "sum dK = 0")
    # weights of each row sum to one, so sum_j dv_j = sum_i dO_i
    _close(dv.sum(axis=1), do.sum(axis=1), 1e-12, 1e-12, "sum dV = sum dO")
    o, _, _ = oracle.attn_fwd(q, k, v, 0.5, lib=lib)
    _close(D, np.sum(do * o, axis=-1), 1e-12, 1e-12, "D = <dO, O>")


# --------------------------------------------------------------------------
# masked (block-sparse) pins


def _random_mask(seed, heads, nbq, nbk, density):
    return (_rng(seed).random((heads, nbq, nbk)) < density).astype(np.uint8)


def pin_masked_all_kept_is_dense(lib):
    q, k, v = _rand(40, 2, 37, 53, 8)
    for bq, bk in ((1, 1), (16, 8), (128, 128)):
        m = np.ones((1, -(-37 // bq), -(-53 // bk)), np.uint8)
        o, lse, _ = oracle.attn_fwd_masked(q, k, v, 0.3, m, bq, bk, lib=lib)
        ro, rl, _ = oracle.attn_fwd(q, k, v, 0.3, lib=lib)
        _close(o, ro, 1e-15, 1e-14, f"all-kept O bq={bq} bk={bk}")
        _close(lse, rl, 1e-15, 1e-14, f"all-kept lse bq={bq} bk={bk}")


def pin_masked_equals_definition_on_kept_keys(lib):
    """Each row equals plain attention (torch float64 softmax / matmul) over
    just the keys its mask blocks keep."""
    cases = [(41, 2, 30, 45, 6, 8, 16, 2), (42, 3, 17, 64, 4, 4, 8, 1), (43, 1, 50, 33, 5, 7, 5, 1)]
    for seed, bh, nq, nk, d, bq, bk, mh in cases:
        q, k, v = _rand(seed, bh, nq, nk, d, qs=1.5)
        m = _random_mask(seed + 100, mh if mh == 1 else bh, -(-nq // bq), -(-nk // bk), 0.55)
        m[:, :, 0] = 1  # every row keeps something
        o, lse, _ = oracle.attn_fwd_masked(q, k, v, 0.4, m, bq, bk, lib=lib)
        for h in range(bh):
            for i in range(nq):
                keep = np.flatnonzero(m[0 if mh == 1 else h, i // bq][np.arange(nk) // bk])
                ro, rl = _torch_fwd(q[h:h + 1, i:i + 1], k[h:h + 1, keep], v[h:h + 1, keep], 0.4)
                _close(o[h, i], ro[0, 0], 1e-13, 1e-12, f"masked O h{h} i{i}")
                _close(lse[h, i], rl[0, 0], 1e-13, 1e-12, f"masked lse h{h} i{i}")


def pin_masked_empty_row_and_single_key(lib):
    q, k, v = _rand(44, 1, 6, 5, 3)
    # bk = 1: mask row block 0 keeps key 3 only, block 1 keeps nothing
    m = np.zeros((1, 2, 5), np.uint8)
    m[0, 0, 3] = 1
    o, lse, _ = oracle.attn_fwd_masked(q, k, v, 0.7, m, 3, 1, lib=lib)
    for i in range(3):
        _close(o[0, i], v[0, 3], 1e-15, 1e-15, "single kept key gives its value")
        _close(lse[0, i], 0.7 * float(q[0, i] @ k[0, 3]), 1e-14, 1e-14, "lse = its score")
    assert np.all(o[0, 3:] == 0.0), "rows with no kept key give O = 0"
    assert np.all(np.isneginf(lse[0, 3:])), "rows with no kept key give lse = -inf"


def pin_masked_block_permutation(lib):
    """Permuting key blocks together with the mask's columns changes nothing."""
    q, k, v = _rand(45, 2, 24, 40, 4)
    m = _random_mask(145, 2, 3, 5, 0.6)
    m[:, :, 1] = 1
    perm = np.array([3, 0, 4, 1, 2])
    kidx = np.concatenate([np.arange(b * 8, b * 8 + 8) for b in perm])
    o1, l1, _ = oracle.attn_fwd_masked(q, k, v, 0.5, m, 8, 8, lib=lib)
    o2, l2, _ = oracle.attn_fwd_masked(q, k[:, kidx], v[:, kidx], 0.5, m[:, :, perm], 8, 8,
                                       lib=lib)
    _close(o2, o1, 1e-14, 1e-13, "key block permutation O")
    _close(l2, l1, 1e-14, 1e-13, "key block permutation lse")


MASKED_PINS = [pin_masked_all_kept_is_dense, pin_masked_equals_definition_on_kept_keys,
               pin_masked_empty_row_and_single_key, pin_masked_block_permutation]


FORWARD_PINS = [pin_golden_forward, pin_torch_library, pin_identity_values_give_weights,
                pin_constant_values, pin_zero_queries_mean_pool, pin_single_key,
                pin_two_keys_logistic, pin_permutations, pin_shift_and_linearity,
                pin_large_scores, pin_large_scores_stream_and_square,
                pin_streaming_equals_direct, pin_square_equals_direct,
                pin_stream_and_square_vs_torch, pin_thread_count]
BACKWARD_PINS = [pin_golden_backward, pin_finite_differences, pin_autograd,
                 pin_gradient_invariants]
ALL_PINS = FORWARD_PINS + MASKED_PINS + BACKWARD_PINS
