/*
 * Float64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU library
 * is compared against; it is compiled into its own shared object
 * (liboracle.so) and may be loaded only by the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark.  It shares no code, header or
 * constant with the HIP library, and the HIP library never calls it.
 *
 * What it computes (page 1, "Attention as a mathematical problem"): for one
 * head with queries q_i, keys k_j and values v_j (rows of Q, K, V),
 *     s_ij = scale * <q_i, k_j>,
 *     p_ij = exp(s_ij) / sum_t exp(s_it),
 *     o_i  = sum_j p_ij v_j.
 * The page writes the score without the 1/sqrt(d) factor, noting only that
 * practical models apply it; here it is the explicit `scale` argument.
 *
 * All arithmetic is IEEE double with libm exp/log, no fast-math.  Batches of
 * heads are independent; `bh` heads are laid out back to back, each row-major
 * [rows, d] with d fastest.  Rows are split over POSIX threads; every output
 * element is produced by exactly one thread in a fixed summation order, so the
 * results do not depend on the thread count.
 *
 * Return value of every entry point: the number of threads used (>= 1), or a
 * negative number on invalid arguments or allocation failure.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* Thread pool helper: run fn(arg, lo, hi) over [0, total) split in T parts. */

typedef void (*range_fn)(void* arg, int64_t lo, int64_t hi, int tid);

typedef struct {
  range_fn fn;
  void* arg;
  int64_t lo, hi;
  int tid;
} range_job;

static void* range_trampoline(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->arg, j->lo, j->hi, j->tid);
  return NULL;
}

static int resolve_threads(int threads, int64_t total) {
  if (threads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    threads = c > 0 ? (int)c : 1;
  }
  if ((int64_t)threads > total) threads = (int)(total > 0 ? total : 1);
  return threads;
}

static int run_parallel(range_fn fn, void* arg, int64_t total, int threads) {
  if (threads <= 1) {
    fn(arg, 0, total, 0);
    return 1;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)threads);
  char* started = (char*)calloc((size_t)threads, 1);
  if (!th || !jobs || !started) {
    free(th);
    free(jobs);
    free(started);
    return -1;
  }
  int64_t per = total / threads, rem = total % threads, start = 0;
  for (int t = 0; t < threads; ++t) {
    int64_t cnt = per + (t < rem ? 1 : 0);
    jobs[t].fn = fn;
    jobs[t].arg = arg;
    jobs[t].lo = start;
    jobs[t].hi = start + cnt;
    jobs[t].tid = t;
    start += cnt;
    /* a thread that cannot be created runs its range here instead */
    if (pthread_create(&th[t], NULL, range_trampoline, &jobs[t]) == 0)
      started[t] = 1;
    else
      fn(arg, jobs[t].lo, jobs[t].hi, t);
  }
  for (int t = 0; t < threads; ++t)
    if (started[t]) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
  free(started);
  return threads;
}

/* ------------------------------------------------------------------------ */
/* Direct definition: three plain loops per query row.                      */

typedef struct {
  const double *Q, *K, *V;
  double *O, *lse;
  int64_t nq, nk, d;
  double scale;
  double** scratch; /* per thread, nk doubles */
} fwd_args;

static void fwd_rows(void* p, int64_t lo, int64_t hi, int tid) {
  fwd_args* a = (fwd_args*)p;
  double* e = a->scratch[tid];
  const int64_t nq = a->nq, nk = a->nk, d = a->d;
  for (int64_t r = lo; r < hi; ++r) {
    const int64_t h = r / nq, i = r % nq;
    const double* q = a->Q + (h * nq + i) * d;
    const double* K = a->K + h * nk * d;
    const double* V = a->V + h * nk * d;
    /* loop 1: scores s_ij = scale * <q_i, k_j> and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
      double dot = 0.0;
      for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + k];
      e[j] = a->scale * dot;
      if (e[j] > m) m = e[j];
    }
    /* loop 2: exponentials shifted by the maximum, and their sum.  The
     * shift is the stability step of page 1, "Softmax without storing the
     * score matrix"; it cancels in the ratio, so the function is unchanged. */
    double ell = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
      e[j] = exp(e[j] - m);
      ell += e[j];
    }
    /* loop 3: o_i = (sum_j e_j v_j) / ell */
    double* o = a->O + (h * nq + i) * d;
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0;
      for (int64_t j = 0; j < nk; ++j) acc += e[j] * V[j * d + k];
      o[k] = acc / ell;
    }
    if (a->lse) a->lse[h * nq + i] = m + log(ell);
  }
}

static double** alloc_scratch(int threads, int64_t n) {
  double** s = (double**)calloc((size_t)threads, sizeof(double*));
  if (!s) return NULL;
  for (int t = 0; t < threads; ++t) {
    s[t] = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!s[t]) {
      for (int u = 0; u < t; ++u) free(s[u]);
      free(s);
      return NULL;
    }
  }
  return s;
}

static void free_scratch(double** s, int threads) {
  if (!s) return;
  for (int t = 0; t < threads; ++t) free(s[t]);
  free(s);
}

/* O[bh, nq, d] and lse[bh, nq] (natural log; may be NULL) from
 * Q[bh, nq, d], K[bh, nk, d], V[bh, nk, d]. */
int oracle_attn_fwd_f64(const double* Q, const double* K, const double* V,
                        double* O, double* lse, int64_t bh, int64_t nq,
                        int64_t nk, int64_t d, double scale, int threads) {
  if (!Q || !K || !V || !O || bh < 0 || nq < 0 || nk < 1 || d < 1) return -1;
  int64_t rows = bh * nq;
  if (rows == 0) return 1;
  threads = resolve_threads(threads, rows);
  fwd_args a = {Q, K, V, O, lse, nq, nk, d, scale, alloc_scratch(threads, nk)};
  if (!a.scratch) return -2;
  int rc = run_parallel(fwd_rows, &a, rows, threads);
  free_scratch(a.scratch, threads);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Masked (block-sparse) definition.  Sparse attention (page 3, "Sparse
 * Attention Extension" and result 2) keeps only some query-key pairs; the
 * page gives lower bounds in terms of the kept entries and no algorithm.
 * Here the kept pairs are given by a block mask: query i and key j interact
 * iff mask[hm][i / bq][j / bk] != 0, with hm = h when mask_heads == bh and
 * hm = 0 when mask_heads == 1 (one mask for every head); the mask is
 * [mask_heads][ceil(nq/bq)][ceil(nk/bk)] bytes.  Each output row is the
 * softmax-weighted average over its kept keys only:
 *     o_i = sum_{j kept} exp(s_ij) v_j / sum_{j kept} exp(s_ij),
 *     lse_i = log sum_{j kept} exp(s_ij).
 * A row with no kept key has no softmax; by convention o_i = 0 and
 * lse_i = -inf.  The same three loops as the direct definition, visiting
 * only kept keys. */

typedef struct {
  const double *Q, *K, *V;
  double *O, *lse;
  int64_t nq, nk, d;
  double scale;
  const uint8_t* mask;
  int64_t mask_heads, bq, bk, nbq, nbk;
  double** scratch; /* per thread, nk doubles */
} masked_args;

static void masked_rows(void* p, int64_t lo, int64_t hi, int tid) {
  masked_args* a = (masked_args*)p;
  double* e = a->scratch[tid];
  const int64_t nq = a->nq, nk = a->nk, d = a->d;
  for (int64_t r = lo; r < hi; ++r) {
    const int64_t h = r / nq, i = r % nq;
    const int64_t hm = a->mask_heads == 1 ? 0 : h;
    const uint8_t* mrow = a->mask + (hm * a->nbq + i / a->bq) * a->nbk;
    const double* q = a->Q + (h * nq + i) * d;
    const double* K = a->K + h * nk * d;
    const double* V = a->V + h * nk * d;
    double* o = a->O + (h * nq + i) * d;
    /* loop 1: scores of the kept keys and their maximum */
    double m = -INFINITY;
    int64_t kept = 0;
    for (int64_t j = 0; j < nk; ++j) {
      if (!mrow[j / a->bk]) continue;
      double dot = 0.0;
      for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + k];
      e[j] = a->scale * dot;
      if (e[j] > m) m = e[j];
      ++kept;
    }
    if (kept == 0) {
      for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
      if (a->lse) a->lse[h * nq + i] = -INFINITY;
      continue;
    }
    /* loop 2: shifted exponentials of the kept keys and their sum */
    double ell = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
      if (!mrow[j / a->bk]) continue;
      e[j] = exp(e[j] - m);
      ell += e[j];
    }
    /* loop 3: o_i = (sum over kept j of e_j v_j) / ell */
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0;
      for (int64_t j = 0; j < nk; ++j)
        if (mrow[j / a->bk]) acc += e[j] * V[j * d + k];
      o[k] = acc / ell;
    }
    if (a->lse) a->lse[h * nq + i] = m + log(ell);
  }
}

int oracle_attn_fwd_masked_f64(const double* Q, const double* K, const double* V,
                               double* O, double* lse, int64_t bh, int64_t nq,
                               int64_t nk, int64_t d, double scale,
                               const uint8_t* mask, int64_t mask_heads,
                               int64_t bq, int64_t bk, int threads) {
  if (!Q || !K || !V || !O || !mask || bh < 0 || nq < 0 || nk < 1 || d < 1 ||
      bq < 1 || bk < 1 || !(mask_heads == 1 || mask_heads == bh))
    return -1;
  int64_t rows = bh * nq;
  if (rows == 0) return 1;
  threads = resolve_threads(threads, rows);
  masked_args a = {Q, K, V, O, lse, nq, nk, d, scale, mask, mask_heads, bq, bk,
                   (nq + bq - 1) / bq, (nk + bk - 1) / bk,
                   alloc_scratch(threads, nk)};
  if (!a.scratch) return -2;
  int rc = run_parallel(masked_rows, &a, rows, threads);
  free_scratch(a.scratch, threads);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Streaming recurrence (page 1, "Softmax without storing the score
 * matrix"): keys are consumed in blocks J of `block` consecutive indices.
 * For each block the running maximum m, normaliser ell and unnormalised
 * output u are updated as
 *     m'   = max(m, max_{j in J} s_j)
 *     ell' = exp(m - m') ell + sum_{j in J} exp(s_j - m')
 *     u'   = exp(m - m') u   + sum_{j in J} exp(s_j - m') v_j
 * starting from m = -inf, ell = 0, u = 0, and finally o = u / ell.  No score
 * outside the current block is kept.  This is the recurrence the fused
 * streaming kernel follows; the oracle of record is the direct definition
 * above, and tests pin this one against it. */

typedef struct {
  const double *Q, *K, *V;
  double *O, *lse;
  int64_t nq, nk, d, block;
  double scale;
  double** scratch; /* per thread: block scores + d accumulators */
} stream_args;

static void stream_rows(void* p, int64_t lo, int64_t hi, int tid) {
  stream_args* a = (stream_args*)p;
  const int64_t nq = a->nq, nk = a->nk, d = a->d, B = a->block;
  double* sblk = a->scratch[tid];
  double* u = sblk + B;
  for (int64_t r = lo; r < hi; ++r) {
    const int64_t h = r / nq, i = r % nq;
    const double* q = a->Q + (h * nq + i) * d;
    const double* K = a->K + h * nk * d;
    const double* V = a->V + h * nk * d;
    double m = -INFINITY, ell = 0.0;
    for (int64_t k = 0; k < d; ++k) u[k] = 0.0;
    for (int64_t j0 = 0; j0 < nk; j0 += B) {
      const int64_t j1 = j0 + B < nk ? j0 + B : nk;
      double mb = -INFINITY;
      for (int64_t j = j0; j < j1; ++j) {
        double dot = 0.0;
        for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + k];
        sblk[j - j0] = a->scale * dot;
        if (sblk[j - j0] > mb) mb = sblk[j - j0];
      }
      const double mnew = m > mb ? m : mb;
      const double alpha = exp(m - mnew); /* exp(-inf) = 0 on the first block */
      ell *= alpha;
      for (int64_t k = 0; k < d; ++k) u[k] *= alpha;
      for (int64_t j = j0; j < j1; ++j) {
        const double e = exp(sblk[j - j0] - mnew);
        ell += e;
        for (int64_t k = 0; k < d; ++k) u[k] += e * V[j * d + k];
      }
      m = mnew;
    }
    double* o = a->O + (h * nq + i) * d;
    for (int64_t k = 0; k < d; ++k) o[k] = u[k] / ell;
    if (a->lse) a->lse[h * nq + i] = m + log(ell);
  }
}

int oracle_attn_fwd_stream_f64(const double* Q, const double* K,
                               const double* V, double* O, double* lse,
                               int64_t bh, int64_t nq, int64_t nk, int64_t d,
                               double scale, int64_t block, int threads) {
  if (!Q || !K || !V || !O || bh < 0 || nq < 0 || nk < 1 || d < 1 || block < 1)
    return -1;
  int64_t rows = bh * nq;
  if (rows == 0) return 1;
  threads = resolve_threads(threads, rows);
  stream_args a = {Q, K, V, O, lse, nq, nk, d, block, scale,
                   alloc_scratch(threads, block + d)};
  if (!a.scratch) return -2;
  int rc = run_parallel(stream_rows, &a, rows, threads);
  free_scratch(a.scratch, threads);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Square-tile schedule for small fast memory (page 1, "Small caches: when
 * storing an intermediate matrix helps"): the score matrix is cut into key
 * tiles of width b.  Step 1 forms each tile's exponentiated scores and keeps
 * them (the intermediate N x N matrix the page says is written to slow
 * memory).  The page does not say how the exponentials are kept finite; the
 * reading used here shifts each (row, tile) by its own maximum m_it and keeps
 * the tile sum ell_it.  Step 2 merges the per-tile statistics with the same
 * rescaling rule as the streaming recurrence:
 *     m_i = max_t m_it,  ell_i = sum_t exp(m_it - m_i) ell_it.
 * Step 3 is the second product: o_i = sum_t (exp(m_it - m_i) / ell_i)
 * sum_{j in t} E_ij v_j.  In exact arithmetic this is the same function as
 * the direct definition. */

typedef struct {
  const double *Q, *K, *V;
  double *O, *lse;
  int64_t nq, nk, d, b;
  double scale;
  double** scratch; /* per thread: nk exponentials + 2*ntiles stats */
} square_args;

static void square_rows(void* p, int64_t lo, int64_t hi, int tid) {
  square_args* a = (square_args*)p;
  const int64_t nq = a->nq, nk = a->nk, d = a->d, b = a->b;
  const int64_t nt = (nk + b - 1) / b;
  double* E = a->scratch[tid];
  double* mt = E + nk;
  double* lt = mt + nt;
  for (int64_t r = lo; r < hi; ++r) {
    const int64_t h = r / nq, i = r % nq;
    const double* q = a->Q + (h * nq + i) * d;
    const double* K = a->K + h * nk * d;
    const double* V = a->V + h * nk * d;
    /* step 1: per key tile, scores, tile maximum, exponentials, tile sum */
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t j0 = t * b, j1 = j0 + b < nk ? j0 + b : nk;
      double m = -INFINITY;
      for (int64_t j = j0; j < j1; ++j) {
        double dot = 0.0;
        for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + k];
        E[j] = a->scale * dot;
        if (E[j] > m) m = E[j];
      }
      double ell = 0.0;
      for (int64_t j = j0; j < j1; ++j) {
        E[j] = exp(E[j] - m);
        ell += E[j];
      }
      mt[t] = m;
      lt[t] = ell;
    }
    /* step 2: merge the tile statistics */
    double m = -INFINITY;
    for (int64_t t = 0; t < nt; ++t)
      if (mt[t] > m) m = mt[t];
    double ell = 0.0;
    for (int64_t t = 0; t < nt; ++t) ell += exp(mt[t] - m) * lt[t];
    /* step 3: second product with per-tile row factors */
    double* o = a->O + (h * nq + i) * d;
    for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t j0 = t * b, j1 = j0 + b < nk ? j0 + b : nk;
      const double f = exp(mt[t] - m) / ell;
      for (int64_t k = 0; k < d; ++k) {
        double acc = 0.0;
        for (int64_t j = j0; j < j1; ++j) acc += E[j] * V[j * d + k];
        o[k] += f * acc;
      }
    }
    if (a->lse) a->lse[h * nq + i] = m + log(ell);
  }
}

int oracle_attn_fwd_square_f64(const double* Q, const double* K,
                               const double* V, double* O, double* lse,
                               int64_t bh, int64_t nq, int64_t nk, int64_t d,
                               double scale, int64_t b, int threads) {
  if (!Q || !K || !V || !O || bh < 0 || nq < 0 || nk < 1 || d < 1 || b < 1)
    return -1;
  int64_t rows = bh * nq;
  if (rows == 0) return 1;
  threads = resolve_threads(threads, rows);
  const int64_t nt = (nk + b - 1) / b;
  square_args a = {Q, K, V, O, lse, nq, nk, d, b, scale,
                   alloc_scratch(threads, nk + 2 * nt)};
  if (!a.scratch) return -2;
  int rc = run_parallel(square_rows, &a, rows, threads);
  free_scratch(a.scratch, threads);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Gradients of the same function.  The pages state the backward problem
 * (page 3, "Methodology", the computational graph of the backward pass) but
 * print no formulas; these are the exact derivatives of o_i with respect to
 * q_i, k_j and v_j given an upstream gradient dO, evaluated row by row:
 *     p_ij  = softmax_j(s_ij),           dP_ij = <dO_i, v_j>,
 *     D_i   = sum_j p_ij dP_ij,          dS_ij = p_ij (dP_ij - D_i),
 *     dq_i  = scale sum_j dS_ij k_j,
 *     dk_j  = scale sum_i dS_ij q_i,     dv_j  = sum_i p_ij dO_i.
 * Rows of one head are split over threads; each thread sums its rows'
 * contributions to dK and dV in a private buffer, and the buffers are added
 * in thread order, so the result is deterministic for a given thread count.
 */

typedef struct {
  const double *Q, *K, *V, *dO;
  double *dQ, *D;
  double **dKp, **dVp; /* per thread [nk, d] partial sums */
  int64_t h, nq, nk, d;
  double scale;
  double** scratch; /* per thread: 2*nk */
} bwd_args;

static void bwd_rows(void* p, int64_t lo, int64_t hi, int tid) {
  bwd_args* a = (bwd_args*)p;
  const int64_t nq = a->nq, nk = a->nk, d = a->d, h = a->h;
  double* P = a->scratch[tid];
  double* dP = P + nk;
  double* dK = a->dKp[tid];
  double* dV = a->dVp[tid];
  const double* K = a->K + h * nk * d;
  const double* V = a->V + h * nk * d;
  for (int64_t i = lo; i < hi; ++i) {
    const double* q = a->Q + (h * nq + i) * d;
    const double* g = a->dO + (h * nq + i) * d;
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
      double dot = 0.0;
      for (int64_t k = 0; k < d; ++k) dot += q[k] * K[j * d + k];
      P[j] = a->scale * dot;
      if (P[j] > m) m = P[j];
    }
    double ell = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
      P[j] = exp(P[j] - m);
      ell += P[j];
    }
    for (int64_t j = 0; j < nk; ++j) P[j] /= ell;
    double Di = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
      double dot = 0.0;
      for (int64_t k = 0; k < d; ++k) dot += g[k] * V[j * d + k];
      dP[j] = dot;
      Di += P[j] * dot;
    }
    if (a->D) a->D[h * nq + i] = Di;
    double* dq = a->dQ + (h * nq + i) * d;
    for (int64_t k = 0; k < d; ++k) dq[k] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
      const double ds = P[j] * (dP[j] - Di);
      for (int64_t k = 0; k < d; ++k) {
        dq[k] += a->scale * ds * K[j * d + k];
        dK[j * d + k] += a->scale * ds * q[k];
        dV[j * d + k] += P[j] * g[k];
      }
    }
  }
}

/* dQ[bh, nq, d], dK[bh, nk, d], dV[bh, nk, d] and optionally D[bh, nq]. */
int oracle_attn_bwd_f64(const double* Q, const double* K, const double* V,
                        const double* dO, double* dQ, double* dK, double* dV,
                        double* D, int64_t bh, int64_t nq, int64_t nk,
                        int64_t d, double scale, int threads) {
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV || bh < 0 || nq < 1 ||
      nk < 1 || d < 1)
    return -1;
  threads = resolve_threads(threads, nq);
  double** scratch = alloc_scratch(threads, 2 * nk);
  double** dKp = alloc_scratch(threads, nk * d);
  double** dVp = alloc_scratch(threads, nk * d);
  if (!scratch || !dKp || !dVp) {
    free_scratch(scratch, threads);
    free_scratch(dKp, threads);
    free_scratch(dVp, threads);
    return -2;
  }
  int rc = 1;
  for (int64_t h = 0; h < bh; ++h) {
    for (int t = 0; t < threads; ++t) {
      memset(dKp[t], 0, sizeof(double) * (size_t)(nk * d));
      memset(dVp[t], 0, sizeof(double) * (size_t)(nk * d));
    }
    bwd_args a = {Q, K, V, dO, dQ, D, dKp, dVp, h, nq, nk, d, scale, scratch};
    rc = run_parallel(bwd_rows, &a, nq, threads);
    if (rc < 0) break;
    double* dk = dK + h * nk * d;
    double* dv = dV + h * nk * d;
    for (int64_t x = 0; x < nk * d; ++x) {
      double sk = 0.0, sv = 0.0;
      for (int t = 0; t < threads; ++t) {
        sk += dKp[t][x];
        sv += dVp[t][x];
      }
      dk[x] = sk;
      dv[x] = sv;
    }
  }
  free_scratch(scratch, threads);
  free_scratch(dKp, threads);
  free_scratch(dVp, threads);
  return rc;
}
