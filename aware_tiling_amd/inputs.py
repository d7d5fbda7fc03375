"""Seeded synthetic inputs for exact attention.

This module holds no attention arithmetic: it only draws tensors.  It is the
one piece shared by the GPU library's tests/benchmark and the float64 oracle's
tests, so both sides see identical numbers.

Recipe (the same for every workload):

* one ``torch.Generator('cpu')`` seeded with the workload's seed;
* tensors drawn in the order Q, K, V, then dO (backward workloads only), each
  ``torch.randn([bh, n, d], dtype=float32)``, i.e. iid N(0, 1);
* bf16 workloads round each fp32 draw to bfloat16 (round to nearest even);
* ``q_mult`` then multiplies Q (4.0 for the large-score workload; a power of
  two, so it is exact in bf16 and its order relative to rounding is moot);
* the scale is ``1/sqrt(d)`` rounded to fp32.

The pages print no dataset or benchmark inputs; these seeded Gaussian tensors
stand in, at the shapes listed in :data:`WORKLOADS`.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    bh: int  # batch x heads
    n: int  # sequence length: keys (and queries unless nq is set)
    d: int  # head dimension
    dtype: str  # "f32" or "bf16" input storage
    seed: int
    q_mult: float = 1.0
    kind: str = "fwd"  # "fwd", "smallcache" or "bwd"
    batch: int = 1
    heads: int = 1
    nq: int = 0  # query rows per head for rectangular workloads (0: n)
    density: float = 1.0  # fraction of 128 x 128 blocks kept (block-sparse workloads)

    @property
    def queries(self) -> int:
        return self.nq or self.n

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    @property
    def fwd_flops(self) -> float:
        """4 nq nk d per head: the two products, mul and add counted apart."""
        return 4.0 * self.queries * self.n * self.d * self.bh


# The five square workloads: a tiny fp32 case, the N=4096/d=64 teaching
# shape, the long-sequence d=128 case with large score ranges, the small-cache
# d=256 case, and the backward case; the backward of the d=256 shape (run by
# the small-cache backward, the one backward built for d=256); then two
# rectangular ones for the key-split forward: single-query decoding of 8
# sequences x 32 heads against a 16384-key cache, and a 1024-query chunk
# against the same cache length; and a block-sparse one at the headline
# shape with a quarter of the 128 x 128 blocks kept (per head, seed + 1000,
# diagonal always kept).
WORKLOADS = {
    w.name: w
    for w in (
        Workload("fwd_f32_h1_n256_d64", 1, 256, 64, "f32", 1, batch=1, heads=1),
        Workload("fwd_bf16_b4h16_n4096_d64", 64, 4096, 64, "bf16", 2, batch=4, heads=16),
        Workload("fwd_bf16_b1h32_n16384_d128_qx4", 32, 16384, 128, "bf16", 3, q_mult=4.0,
                 batch=1, heads=32),
        Workload("smallcache_bf16_b1h8_n4096_d256", 8, 4096, 256, "bf16", 4,
                 kind="smallcache", batch=1, heads=8),
        Workload("bwd_bf16_b2h16_n4096_d128", 32, 4096, 128, "bf16", 5, kind="bwd",
                 batch=2, heads=16),
        Workload("bwd_smallcache_bf16_b1h8_n4096_d256", 8, 4096, 256, "bf16", 8, kind="bwd",
                 batch=1, heads=8),
        Workload("sparse_bf16_b1h32_n16384_d128_keep25", 32, 16384, 128, "bf16", 9,
                 kind="sparse", batch=1, heads=32, density=0.25),
        Workload("decode_bf16_b8h32_q1_k16384_d128", 256, 16384, 128, "bf16", 6, kind="splitk",
                 batch=8, heads=32, nq=1),
        Workload("chunk_bf16_b1h32_q1024_k16384_d128", 32, 16384, 128, "bf16", 7,
                 kind="splitk", batch=1, heads=32, nq=1024),
    )
}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(bh: int, n: int, d: int, dtype: str = "bf16", seed: int = 0,
                q_mult: float = 1.0, with_do: bool = False, nk: int | None = None):
    """Draw (Q, K, V[, dO]) on the CPU following the recipe above.

    ``nk`` (default ``n``) allows a different key count for rectangular
    cases; Q and dO have ``n`` rows, K and V have ``nk``.
    """
    nk = n if nk is None else nk
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((bh, n, d), dtype=torch.float32, generator=g)
    k = torch.randn((bh, nk, d), dtype=torch.float32, generator=g)
    v = torch.randn((bh, nk, d), dtype=torch.float32, generator=g)
    out = [q, k, v]
    if with_do:
        out.append(torch.randn((bh, n, d), dtype=torch.float32, generator=g))
    tdt = TORCH_DTYPES[dtype]
    out = [t.to(tdt) for t in out]
    if q_mult != 1.0:
        out[0] = (out[0] * q_mult).to(tdt)
    return tuple(out)


def make_block_mask(heads: int, nb: int, density: float, seed: int,
                    keep_diagonal: bool = True) -> torch.Tensor:
    """A seeded random block mask [heads, nb, nb] (uint8, 1 = kept): each
    block kept independently with probability ``density`` (one
    ``torch.rand`` draw per block from a CPU generator seeded with ``seed``),
    plus the diagonal blocks when ``keep_diagonal`` (so no query row is left
    without keys)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    m = (torch.rand((heads, nb, nb), generator=g) < density).to(torch.uint8)
    if keep_diagonal:
        idx = torch.arange(nb)
        m[:, idx, idx] = 1
    return m


def workload_inputs(w: Workload):
    return make_inputs(w.bh, w.queries, w.d, w.dtype, w.seed, w.q_mult,
                       with_do=(w.kind == "bwd"), nk=w.n)
