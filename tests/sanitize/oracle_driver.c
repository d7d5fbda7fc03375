/* Test driver for the oracle under AddressSanitizer and UBSan (host only).
 *
 * Runs every oracle entry point on small ragged shapes with buffers of
 * exactly the documented sizes (so any out-of-bounds access is reported),
 * with one and with three threads, and checks the results against each
 * other: the streaming and square-tile recurrences and an all-kept block
 * mask must reproduce the direct definition to 1e-12, and one thread must
 * agree with three bit for bit.  Exit status 0 when everything holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_fwd_f64(const double*, const double*, const double*, double*, double*,
                        int64_t, int64_t, int64_t, int64_t, double, int);
int oracle_attn_fwd_masked_f64(const double*, const double*, const double*, double*,
                               double*, int64_t, int64_t, int64_t, int64_t, double,
                               const uint8_t*, int64_t, int64_t, int64_t, int);
int oracle_attn_fwd_stream_f64(const double*, const double*, const double*, double*,
                               double*, int64_t, int64_t, int64_t, int64_t, double,
                               int64_t, int);
int oracle_attn_fwd_square_f64(const double*, const double*, const double*, double*,
                               double*, int64_t, int64_t, int64_t, int64_t, double,
                               int64_t, int);
int oracle_attn_bwd_f64(const double*, const double*, const double*, const double*,
                        double*, double*, double*, double*, int64_t, int64_t, int64_t,
                        int64_t, double, int);

static uint64_t state = 88172645463325252ull;
static double rnd(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double* filled(int64_t count) {
  double* p = malloc((size_t)count * sizeof(double));
  for (int64_t i = 0; i < count; ++i) p[i] = rnd();
  return p;
}
static double maxdiff(const double* a, const double* b, int64_t count) {
  double m = 0.0;
  for (int64_t i = 0; i < count; ++i) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

static int fails = 0;
static void expect(int ok, const char* what, int64_t bh, int64_t nq, int64_t nk, int64_t d) {
  if (!ok) {
    fprintf(stderr, "FAIL %s bh=%lld nq=%lld nk=%lld d=%lld\n", what, (long long)bh,
            (long long)nq, (long long)nk, (long long)d);
    ++fails;
  }
}

static void run_case(int64_t bh, int64_t nq, int64_t nk, int64_t d) {
  const double s = 1.0 / sqrt((double)d);
  double *Q = filled(bh * nq * d), *K = filled(bh * nk * d), *V = filled(bh * nk * d);
  double* dO = filled(bh * nq * d);
  const int64_t no = bh * nq * d, nl = bh * nq;
  double *O1 = malloc(no * sizeof(double)), *L1 = malloc(nl * sizeof(double));
  double *O3 = malloc(no * sizeof(double)), *L3 = malloc(nl * sizeof(double));
  double *O = malloc(no * sizeof(double)), *L = malloc(nl * sizeof(double));
  expect(oracle_attn_fwd_f64(Q, K, V, O1, L1, bh, nq, nk, d, s, 1) > 0, "fwd 1 thread", bh, nq, nk, d);
  expect(oracle_attn_fwd_f64(Q, K, V, O3, L3, bh, nq, nk, d, s, 3) > 0, "fwd 3 threads", bh, nq, nk, d);
  expect(memcmp(O1, O3, no * sizeof(double)) == 0 && memcmp(L1, L3, nl * sizeof(double)) == 0,
         "fwd threads bitwise", bh, nq, nk, d);
  const int64_t blocks[] = {1, 7, 64, nk};
  for (int i = 0; i < 4; ++i) {
    expect(oracle_attn_fwd_stream_f64(Q, K, V, O, L, bh, nq, nk, d, s, blocks[i], 3) > 0,
           "stream", bh, nq, nk, d);
    expect(maxdiff(O, O1, no) < 1e-12 && maxdiff(L, L1, nl) < 1e-12, "stream = direct", bh, nq,
           nk, d);
    expect(oracle_attn_fwd_square_f64(Q, K, V, O, L, bh, nq, nk, d, s, blocks[i], 3) > 0,
           "square", bh, nq, nk, d);
    expect(maxdiff(O, O1, no) < 1e-12 && maxdiff(L, L1, nl) < 1e-12, "square = direct", bh, nq,
           nk, d);
  }
  const int64_t bq = 16, bk = 32, nbq = (nq + bq - 1) / bq, nbk = (nk + bk - 1) / bk;
  uint8_t* mask = malloc((size_t)(bh * nbq * nbk));
  memset(mask, 1, (size_t)(bh * nbq * nbk));
  expect(oracle_attn_fwd_masked_f64(Q, K, V, O, L, bh, nq, nk, d, s, mask, bh, bq, bk, 3) > 0,
         "masked", bh, nq, nk, d);
  expect(maxdiff(O, O1, no) < 1e-12 && maxdiff(L, L1, nl) < 1e-12, "all-kept mask = direct",
         bh, nq, nk, d);
  for (int64_t i = 0; i < bh * nbq * nbk; ++i) mask[i] = (uint8_t)(rnd() > 0.0);
  expect(oracle_attn_fwd_masked_f64(Q, K, V, O, L, bh, nq, nk, d, s, mask, bh, bq, bk, 3) > 0,
         "masked random", bh, nq, nk, d);
  free(mask);
  if (nq == nk) {
    double *dQ = malloc(no * sizeof(double)), *dK = malloc(no * sizeof(double));
    double *dV = malloc(no * sizeof(double)), *D = malloc(nl * sizeof(double));
    double *dQ1 = malloc(no * sizeof(double)), *dK1 = malloc(no * sizeof(double));
    double *dV1 = malloc(no * sizeof(double));
    expect(oracle_attn_bwd_f64(Q, K, V, dO, dQ, dK, dV, D, bh, nq, nk, d, s, 3) > 0, "bwd", bh,
           nq, nk, d);
    expect(oracle_attn_bwd_f64(Q, K, V, dO, dQ1, dK1, dV1, NULL, bh, nq, nk, d, s, 1) > 0,
           "bwd 1 thread", bh, nq, nk, d);
    expect(maxdiff(dQ, dQ1, no) < 1e-12 && maxdiff(dK, dK1, no) < 1e-12 &&
               maxdiff(dV, dV1, no) < 1e-12,
           "bwd threads agree", bh, nq, nk, d);
    free(dQ); free(dK); free(dV); free(D); free(dQ1); free(dK1); free(dV1);
  }
  free(Q); free(K); free(V); free(dO); free(O1); free(L1); free(O3); free(L3); free(O); free(L);
}

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {1, 5, 5, 3}, {2, 33, 33, 8}, {1, 17, 70, 16},
                               {3, 65, 65, 5}, {1, 100, 37, 64}};
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
    run_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3]);
  if (fails) return 1;
  printf("oracle under sanitizers: all cases passed\n");
  return 0;
}
