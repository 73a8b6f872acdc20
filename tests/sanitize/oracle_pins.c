/*
 * oracle_pins.c -- the oracle's core pins as a plain C program, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer together with oracle/linattn_oracle.c (tests/test_sanitizers.py).
 * Every oracle entry point runs on the shapes the Python pins use (and the empty ones), so an
 * out-of-bounds access, a leak or undefined behaviour in the oracle stops the program.
 *
 * What is checked ("Efficient Transformers: Linear Attention and Flash Attention"):
 *   - "Worked example: the reassociation trick, by hand": with phi(x) = x, K^T V = [[3,2],[2,4]],
 *     the key sum (4,5), outputs (3/4,1/2), (2/5,4/5), (5/9,2/3) by both evaluation orders, and
 *     the causal rows (1,0), (1/4,3/4), (5/9,2/3) derived from the same numbers;
 *   - eq. Attention_i: the linear order equals the explicit n x n order (elu + 1, random inputs);
 *   - "The recurrent view": recurrence = masked quadratic order = chunked regrouping at several
 *     chunk sizes (ragged tails included), decode steps from the empty state = recurrence, the
 *     state after n tokens = the accumulated sums, rows by the definition = the full forms.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_noncausal_linear(const double*, const double*, const double*, double*, int64_t, int64_t,
                          int64_t, int, double*, double*);
void orc_quadratic(const double*, const double*, const double*, double*, int64_t, int64_t, int64_t,
                   int, int, double*);
void orc_causal_recurrent(const double*, const double*, const double*, double*, int64_t, int64_t,
                          int64_t, int, const double*, const double*, double*, double*);
void orc_causal_chunked(const double*, const double*, const double*, double*, int64_t, int64_t,
                        int64_t, int64_t, int);
void orc_decode_step(const double*, const double*, const double*, double*, double*, double*,
                     int64_t, int64_t, int);
void orc_rows(const double*, const double*, const double*, double*, int64_t, int64_t,
              const int64_t*, int64_t, int, int);
void orc_phi_rows(const double*, double*, int64_t, int);
void orc_state_accumulate(const double*, const double*, double*, double*, int64_t, int64_t, int64_t,
                          int);

#define ELU1 0
#define IDENTITY 1

static int failures = 0;

static void expect_close(const char* what, const double* a, const double* b, int64_t count, double tol) {
  double worst = 0.0;
  for (int64_t i = 0; i < count; ++i) {
    const double e = fabs(a[i] - b[i]) / (fabs(b[i]) > 1.0 ? fabs(b[i]) : 1.0);
    if (!(e <= worst)) worst = e; /* NaN counts as a failure */
  }
  if (!(worst <= tol)) {
    printf("FAIL %s: worst error %.3e (tol %.1e)\n", what, worst, tol);
    ++failures;
  }
}

/* xorshift doubles in [-2, 2): inputs only, no arithmetic of the method */
static uint64_t rng_state = 88172645463325252ull;
static double uniform(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0 * 4.0 - 2.0;
}

static double* fresh(int64_t count) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(count > 0 ? count : 1));
  for (int64_t i = 0; i < count; ++i) p[i] = uniform();
  return p;
}

static void worked_example(void) {
  const double Q[6] = {1, 0, 0, 1, 1, 1}, K[6] = {2, 1, 1, 3, 1, 1}, V[6] = {1, 0, 0, 1, 1, 1};
  const double printed[6] = {3.0 / 4, 1.0 / 2, 2.0 / 5, 4.0 / 5, 5.0 / 9, 2.0 / 3};
  const double causal[6] = {1, 0, 1.0 / 4, 3.0 / 4, 5.0 / 9, 2.0 / 3};
  const double KtV[4] = {3, 2, 2, 4}, ksum[2] = {4, 5};
  double out[6], kv[4], z[2], w[9];
  orc_noncausal_linear(Q, K, V, out, 1, 3, 2, IDENTITY, kv, z);
  expect_close("worked example, linear order", out, printed, 6, 1e-15);
  expect_close("worked example, K^T V", kv, KtV, 4, 0.0);
  expect_close("worked example, key sum", z, ksum, 2, 0.0);
  orc_quadratic(Q, K, V, out, 1, 3, 2, 0, IDENTITY, w);
  const double scores[9] = {2, 1, 1, 1, 3, 1, 3, 4, 2};
  expect_close("worked example, Q K^T", w, scores, 9, 0.0);
  expect_close("worked example, quadratic order", out, printed, 6, 1e-15);
  orc_causal_recurrent(Q, K, V, out, 1, 3, 2, IDENTITY, NULL, NULL, NULL, NULL);
  expect_close("worked example, causal recurrence", out, causal, 6, 1e-15);
  orc_quadratic(Q, K, V, out, 1, 3, 2, 1, IDENTITY, NULL);
  expect_close("worked example, causal quadratic", out, causal, 6, 1e-15);
}

static void forms_agree(int64_t BH, int64_t n, int64_t d) {
  const int64_t e = BH * n * d;
  double *q = fresh(e), *k = fresh(e), *v = fresh(e);
  double *a = fresh(e), *b = fresh(e);
  char what[96];
  /* non-causal: linear order = quadratic order */
  orc_noncausal_linear(q, k, v, a, BH, n, d, ELU1, NULL, NULL);
  orc_quadratic(q, k, v, b, BH, n, d, 0, ELU1, NULL);
  snprintf(what, sizeof what, "linear = quadratic (BH=%lld n=%lld d=%lld)", (long long)BH, (long long)n, (long long)d);
  expect_close(what, a, b, e, 1e-12);
  /* causal: recurrence = masked quadratic = chunked regroupings */
  double *Sf = fresh(BH * d * d), *zf = fresh(BH * d);
  orc_causal_recurrent(q, k, v, a, BH, n, d, ELU1, NULL, NULL, Sf, zf);
  orc_quadratic(q, k, v, b, BH, n, d, 1, ELU1, NULL);
  snprintf(what, sizeof what, "recurrence = masked quadratic (n=%lld d=%lld)", (long long)n, (long long)d);
  expect_close(what, a, b, e, 1e-12);
  const int64_t chunks[5] = {1, 3, 16, 64, 1000};
  for (int c = 0; c < 5; ++c) {
    orc_causal_chunked(q, k, v, b, BH, n, d, chunks[c], ELU1);
    snprintf(what, sizeof what, "recurrence = chunked C=%lld (n=%lld)", (long long)chunks[c], (long long)n);
    expect_close(what, a, b, e, 1e-12);
  }
  /* the final state = the accumulated sums of every token */
  double* S = (double*)calloc((size_t)(BH * d * d > 0 ? BH * d * d : 1), sizeof(double));
  double* z = (double*)calloc((size_t)(BH * d > 0 ? BH * d : 1), sizeof(double));
  orc_state_accumulate(k, v, S, z, BH, n, d, ELU1);
  expect_close("final state S = accumulated sums", Sf, S, BH * d * d, 1e-12);
  expect_close("final state z = accumulated sums", zf, z, BH * d, 1e-12);
  /* decode steps from the empty state = the recurrence */
  memset(S, 0, sizeof(double) * (size_t)(BH * d * d));
  memset(z, 0, sizeof(double) * (size_t)(BH * d));
  double *qt = fresh(BH * d), *kt = fresh(BH * d), *vt = fresh(BH * d), *ot = fresh(BH * d);
  for (int64_t t = 0; t < n; ++t) {
    for (int64_t h = 0; h < BH; ++h)
      for (int64_t x = 0; x < d; ++x) {
        qt[h * d + x] = q[(h * n + t) * d + x];
        kt[h * d + x] = k[(h * n + t) * d + x];
        vt[h * d + x] = v[(h * n + t) * d + x];
      }
    orc_decode_step(qt, kt, vt, S, z, ot, BH, d, ELU1);
    for (int64_t h = 0; h < BH; ++h)
      for (int64_t x = 0; x < d; ++x) b[(h * n + t) * d + x] = ot[h * d + x];
  }
  snprintf(what, sizeof what, "decode steps = recurrence (n=%lld)", (long long)n);
  expect_close(what, a, b, e, 1e-12);
  /* single rows by the definition, for the first head */
  if (n > 0) {
    double* pk = fresh(n * d);
    orc_phi_rows(k, pk, n * d, ELU1);
    const int64_t rows[3] = {0, n / 2, n - 1};
    double* r = fresh(3 * d);
    orc_rows(q, pk, v, r, n, d, rows, 3, 1, ELU1);
    for (int i = 0; i < 3; ++i) expect_close("causal rows = recurrence", r + i * d, a + rows[i] * d, d, 1e-12);
    orc_rows(q, pk, v, r, n, d, rows, 3, 0, ELU1);
    orc_noncausal_linear(q, k, v, b, BH, n, d, ELU1, NULL, NULL);
    for (int i = 0; i < 3; ++i) expect_close("rows = linear order", r + i * d, b + rows[i] * d, d, 1e-12);
    free(pk);
    free(r);
  }
  free(q); free(k); free(v); free(a); free(b); free(Sf); free(zf); free(S); free(z);
  free(qt); free(kt); free(vt); free(ot);
}

int main(void) {
  worked_example();
  const int64_t shapes[][3] = {{1, 0, 8}, {2, 1, 4}, {1, 2, 1}, {3, 5, 3}, {2, 70, 8}, {1, 129, 16}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) forms_agree(shapes[s][0], shapes[s][1], shapes[s][2]);
  if (failures) {
    printf("%d pin(s) failed\n", failures);
    return 1;
  }
  printf("oracle pins OK under the sanitizers\n");
  return 0;
}
