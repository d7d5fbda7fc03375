"""Float64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  This package is the checker the GPU library is
compared against.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the library under ``aware_tiling_amd``
never does, and the two share no code (the only thing they share is the
seeded input generator, which holds none of the method's arithmetic).

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double, libm
``exp``/``log``, POSIX threads over query rows).  This module compiles it with
gcc into ``liboracle.so`` next to the source and wraps it with ctypes.  Inputs
are numpy arrays of any float dtype; they are widened to float64 exactly
(bf16 and fp32 values are representable in double), so the oracle sees the
same numbers the GPU sees.

Entry points (all shapes ``[bh, rows, d]``, d fastest):

* :func:`attn_fwd` -- the direct definition of page 1, "Attention as a
  mathematical problem": ``O = softmax(scale * Q K^T) V`` row by row, plus the
  natural-log log-sum-exp of each row's scaled scores.
* :func:`attn_fwd_stream` -- the blockwise running-maximum recurrence of
  page 1, "Softmax without storing the score matrix".
* :func:`attn_fwd_square` -- the square-tile schedule of page 1, "Small caches:
  when storing an intermediate matrix helps" (per-tile exponentials, merged
  statistics, second product).
* :func:`attn_fwd_masked` -- the direct definition restricted to the
  query-key pairs a block mask keeps (page 3's sparse attention), rows with
  no kept key giving O = 0 and lse = -inf.
* :func:`attn_bwd` -- exact gradients dQ, dK, dV of the same function for an
  upstream gradient dO (page 3 states the backward problem; the formulas are
  ordinary calculus, written out in ``attn_oracle.c``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_F64P = ctypes.POINTER(ctypes.c_double)


def build(src: str = _SRC, out: str = _SO) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into a shared object."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-pthread", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared object."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = _bind(ctypes.CDLL(_SO))
    return _lib


def _bind(lib):
    i64, dbl, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.oracle_attn_fwd_f64.argtypes = [_F64P] * 5 + [i64] * 4 + [dbl, cint]
    lib.oracle_attn_fwd_stream_f64.argtypes = [_F64P] * 5 + [i64] * 4 + [dbl, i64, cint]
    lib.oracle_attn_fwd_square_f64.argtypes = [_F64P] * 5 + [i64] * 4 + [dbl, i64, cint]
    lib.oracle_attn_bwd_f64.argtypes = [_F64P] * 8 + [i64] * 4 + [dbl, cint]
    lib.oracle_attn_fwd_masked_f64.argtypes = ([_F64P] * 5 + [i64] * 4 +
                                               [dbl, ctypes.c_void_p, i64, i64, i64, cint])
    for f in (lib.oracle_attn_fwd_f64, lib.oracle_attn_fwd_stream_f64,
              lib.oracle_attn_fwd_square_f64, lib.oracle_attn_bwd_f64,
              lib.oracle_attn_fwd_masked_f64):
        f.restype = cint
    return lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().to("cpu")
        import torch  # local: only needed for torch inputs

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_F64P)


def _shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("Q, K, V must be [bh, rows, d]")
    bh, nq, d = q.shape
    if k.shape[0] != bh or v.shape[0] != bh or k.shape[2] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: Q{q.shape} K{k.shape} V{v.shape}")
    return bh, nq, k.shape[1], d


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")
    return rc


def attn_fwd(q, k, v, scale: float, threads: int = 0, lib=None):
    """Direct definition. Returns (O [bh,nq,d], lse [bh,nq], threads_used)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, nq, nk, d = _shapes(q, k, v)
    o = np.empty((bh, nq, d))
    lse = np.empty((bh, nq))
    lib = lib or load()
    t = _check(lib.oracle_attn_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       bh, nq, nk, d, float(scale), int(threads)), "fwd")
    return o, lse, t


def attn_fwd_masked(q, k, v, scale: float, mask, bq: int, bk: int, threads: int = 0,
                    lib=None):
    """Definition over the pairs a block mask keeps.  ``mask`` is
    [mask_heads, ceil(nq/bq), ceil(nk/bk)] (nonzero = kept), mask_heads 1 or
    bh.  Returns (O, lse, threads_used); rows with no kept key give O = 0,
    lse = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, nq, nk, d = _shapes(q, k, v)
    if hasattr(mask, "detach"):
        mask = mask.detach().to("cpu").numpy()
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    nbq, nbk = -(-nq // bq), -(-nk // bk)
    if m.ndim != 3 or m.shape[1:] != (nbq, nbk) or m.shape[0] not in (1, bh):
        raise ValueError(f"mask shape {m.shape} does not match ({bh} or 1, {nbq}, {nbk})")
    o = np.empty((bh, nq, d))
    lse = np.empty((bh, nq))
    lib = lib or load()
    t = _check(lib.oracle_attn_fwd_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              bh, nq, nk, d, float(scale),
                                              m.ctypes.data_as(ctypes.c_void_p), m.shape[0],
                                              int(bq), int(bk), int(threads)), "fwd_masked")
    return o, lse, t


def attn_fwd_stream(q, k, v, scale: float, block: int, threads: int = 0, lib=None):
    """Running-maximum recurrence over key blocks of ``block`` keys."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, nq, nk, d = _shapes(q, k, v)
    o = np.empty((bh, nq, d))
    lse = np.empty((bh, nq))
    lib = lib or load()
    t = _check(lib.oracle_attn_fwd_stream_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              bh, nq, nk, d, float(scale), int(block),
                                              int(threads)), "fwd_stream")
    return o, lse, t


def attn_fwd_square(q, k, v, scale: float, b: int, threads: int = 0, lib=None):
    """Square-tile schedule with key tiles of width ``b``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, nq, nk, d = _shapes(q, k, v)
    o = np.empty((bh, nq, d))
    lse = np.empty((bh, nq))
    lib = lib or load()
    t = _check(lib.oracle_attn_fwd_square_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              bh, nq, nk, d, float(scale), int(b),
                                              int(threads)), "fwd_square")
    return o, lse, t


def attn_bwd(q, k, v, do, scale: float, threads: int = 0, lib=None):
    """Exact gradients. Returns (dQ, dK, dV, D, threads_used); D_i = <dO_i, o_i>."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    bh, nq, nk, d = _shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have Q's shape")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    D = np.empty((bh, nq))
    lib = lib or load()
    t = _check(lib.oracle_attn_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(D), bh, nq, nk, d,
                                       float(scale), int(threads)), "bwd")
    return dq, dk, dv, D, t
