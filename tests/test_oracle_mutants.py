"""The pins catch plausible slips in the oracle (CPU only).

Each mutant is a copy of oracle/attn_oracle.c with one deliberate mistake of
the kind that hides easily (a dropped term, a flipped sign, a wrong index, a
missing rescale).  It is compiled with gcc into a temporary shared object and
the whole pin battery of tests/oracle_pins.py runs against it; at least one
pin must fail.  Every mutant keeps its memory accesses in bounds.
"""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

DOT_K = "for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + k];"
DOT_K_REV = "for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + (d - 1 - k)];"

# (id, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("direct_scale_dropped", "e[j] = a->scale * dot;", "e[j] = dot;", 0),
    ("direct_key_columns_reversed", DOT_K, DOT_K_REV, 0),
    ("direct_exponent_sign", "e[j] = exp(e[j] - m);", "e[j] = exp(m - e[j]);", 0),
    ("direct_sum_drops_first_key", "ell += e[j];", "ell += (j > 0) ? e[j] : 0.0;", 0),
    ("direct_value_columns_reversed", "acc += e[j] * V[j * d + k];",
     "acc += e[j] * V[j * d + (d - 1 - k)];", 0),
    ("direct_output_skips_first_key",
     "for (int64_t j = 0; j < nk; ++j) acc += e[j] * V[j * d + k];",
     "for (int64_t j = 1; j < nk; ++j) acc += e[j] * V[j * d + k];", 0),
    ("direct_lse_without_max", "a->lse[h * nq + i] = m + log(ell);",
     "a->lse[h * nq + i] = log(ell);", 0),
    ("masked_row_block_uses_key_block_size",
     "a->mask + (hm * a->nbq + i / a->bq) * a->nbk", "a->mask + (hm * a->nbq + i / a->bk) * a->nbk",
     0),
    ("masked_mask_shared_by_all_heads", "const int64_t hm = a->mask_heads == 1 ? 0 : h;",
     "const int64_t hm = 0;", 0),
    ("masked_sum_over_dropped_keys",
     "      if (!mrow[j / a->bk]) continue;\n      e[j] = exp(e[j] - m);",
     "      e[j] = mrow[j / a->bk] ? exp(e[j] - m) : exp(-1.0);", 0),
    ("masked_empty_row_lse_zero", "if (a->lse) a->lse[h * nq + i] = -INFINITY;",
     "if (a->lse) a->lse[h * nq + i] = 0.0;", 0),
    ("stream_sum_not_rescaled", "ell *= alpha;", "", 0),
    ("stream_output_not_rescaled", "for (int64_t k = 0; k < d; ++k) u[k] *= alpha;", "", 0),
    ("stream_max_not_carried", "const double mnew = m > mb ? m : mb;",
     "const double mnew = mb;", 0),
    ("stream_scale_dropped", "sblk[j - j0] = a->scale * dot;", "sblk[j - j0] = dot;", 0),
    ("square_merge_ignores_tile_max", "ell += exp(mt[t] - m) * lt[t];", "ell += lt[t];", 0),
    ("square_factor_ignores_tile_max", "const double f = exp(mt[t] - m) / ell;",
     "const double f = 1.0 / ell;", 0),
    ("square_tile_max_reset", "if (E[j] > m) m = E[j];", "m = E[j];", 0),
    ("bwd_D_sign", "const double ds = P[j] * (dP[j] - Di);",
     "const double ds = P[j] * (dP[j] + Di);", 0),
    ("bwd_dK_scale_dropped", "dK[j * d + k] += a->scale * ds * q[k];",
     "dK[j * d + k] += ds * q[k];", 0),
    ("bwd_dV_columns_reversed", "dV[j * d + k] += P[j] * g[k];",
     "dV[j * d + k] += P[j] * g[d - 1 - k];", 0),
    ("bwd_dQ_uses_value", "dq[k] += a->scale * ds * K[j * d + k];",
     "dq[k] += a->scale * ds * V[j * d + k];", 0),
    ("bwd_weights_not_normalised", "for (int64_t j = 0; j < nk; ++j) P[j] /= ell;", "", 0),
    ("bwd_thread_partials_dropped", "sk += dKp[t][x];", "sk = dKp[t][x];", 0),
    ("bwd_dP_transposed", "for (int64_t k = 0; k < d; ++k) dot += g[k] * V[j * d + k];",
     "for (int64_t k = 0; k < d; ++k) dot += g[k] * V[j * d + (d - 1 - k)];", 0),
]


def _mutate(src: str, old: str, new: str, occ: int) -> str:
    pos = -1
    for _ in range(occ + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation site not found: {old!r}"
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("mid,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(mid, old, new, occ, tmp_path):
    src = open(SRC).read()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    cfile = tmp_path / f"{mid}.c"
    cfile.write_text(mutated)
    so = oracle.build(str(cfile), str(tmp_path / f"lib{mid}.so"))
    lib = oracle.load(so)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            failures.append(f"{pin.__name__}: {e}")
            break
    assert failures, f"mutant {mid} passed every pin"
