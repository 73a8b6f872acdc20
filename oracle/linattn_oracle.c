/*
 * linattn_oracle.c -- plain, slow, single-threaded fp64 CPU oracle for kernelized
 * linear attention with the feature map phi(x) = elu(x) + 1.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this code: only the
 * test suite, the smoke check and the CPU-baseline leg of bench.py load it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it follows (page titles and sections; no code from the pages is reproduced):
 *   [G12]  "Efficient Transformers: Linear Attention and Flash Attention"
 *          (aicomputerinstitute.com, grade 12), sections
 *          - "Linear attention: reordering the matmuls, not shrinking them": the output of
 *            query i is phi(Q_i).sum_j phi(K_j)V_j^T divided by phi(Q_i).sum_j phi(K_j),
 *            with phi = elu + 1 (eq. Attention_i);
 *          - "Worked example: the reassociation trick, by hand": the quadratic (standard)
 *            and the linear (reassociated) evaluation order give the same result;
 *          - "The recurrent view: attention as an RNN": S_t = S_{t-1} + phi(K_t)V_t^T,
 *            z_t = z_{t-1} + phi(K_t), output phi(Q_t).S_t / phi(Q_t).z_t;
 *          - Active recall A4 (phi must be non-negative) and A5 (fixed-size state).
 *
 * Conventions.  Every array is contiguous row-major double.  A batch of heads is laid out
 * [BH][n][d]; the per-head state S is [d][d] with S[a][c] = sum_j phi(k_j)[a] * v_j[c]
 * (feature row a, value column c), z is [d].  The feature dimension D equals d because
 * phi is elementwise.  All sums run in ascending index order.  No blocking, fusion or
 * reordering is done beyond what each form's definition states.
 *
 * Readings of points the pages leave open (each is the plainest reading):
 *   - elu uses alpha = 1, so phi(x) = x + 1 for x > 0 and exp(x) for x <= 0
 *     (elu(x) + 1 = (exp(x) - 1) + 1 = exp(x) there, evaluated as exp(x) directly);
 *   - no 1/sqrt(d) scaling and no epsilon in the denominator: the formula has neither;
 *   - the causal mask is inclusive (key j contributes to query i when j <= i);
 *   - a decode step first folds the new (k, v) into the state, then reads it with q.
 *
 * Parity pins (see tests/test_oracle_pins.py): the worked example's printed values, the
 * linear form against the quadratic form, the recurrence against the masked quadratic
 * form, positivity, the convex-combination bound, the ones vector, causal special cases,
 * decode against causal, permutation invariance and linearity in V.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Feature maps.  ORC_PHI_IDENTITY exists only to reproduce the hand-worked example of
 * [G12] "Worked example", which uses phi(x) = x on non-negative inputs. */
#define ORC_PHI_ELU1 0
#define ORC_PHI_IDENTITY 1

/* phi(x) = elu(x) + 1 with alpha = 1 ([G12] "Linear attention", feature map of
 * Katharopoulos et al.). */
double orc_phi(double x, int map) {
  if (map == ORC_PHI_IDENTITY) return x;
  if (x > 0.0) return x + 1.0;
  return exp(x);
}

/* Non-causal, linear (reassociated) order: build KV = phi(K)^T V and z = sum_j phi(K_j)
 * once per head, then out_i = phi(Q_i) KV / phi(Q_i) z  ([G12] eq. Attention_i and the
 * "Linear path" of the worked example).  kv_out ([BH][d][d]) and z_out ([BH][d]) may be
 * NULL; when given they receive the per-head aggregates. */
void orc_noncausal_linear(const double* q, const double* k, const double* v, double* out,
                          int64_t BH, int64_t n, int64_t d, int map, double* kv_out,
                          double* z_out) {
  double* KV = (double*)malloc(sizeof(double) * (size_t)(d * d));
  double* z = (double*)malloc(sizeof(double) * (size_t)d);
  double* fq = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t h = 0; h < BH; ++h) {
    const double* Q = q + h * n * d;
    const double* K = k + h * n * d;
    const double* V = v + h * n * d;
    double* O = out + h * n * d;
    for (int64_t a = 0; a < d; ++a) {
      z[a] = 0.0;
      for (int64_t c = 0; c < d; ++c) KV[a * d + c] = 0.0;
    }
    for (int64_t j = 0; j < n; ++j) {
      for (int64_t a = 0; a < d; ++a) {
        double fk = orc_phi(K[j * d + a], map);
        z[a] += fk;
        for (int64_t c = 0; c < d; ++c) KV[a * d + c] += fk * V[j * d + c];
      }
    }
    for (int64_t i = 0; i < n; ++i) {
      for (int64_t a = 0; a < d; ++a) fq[a] = orc_phi(Q[i * d + a], map);
      double den = 0.0;
      for (int64_t a = 0; a < d; ++a) den += fq[a] * z[a];
      for (int64_t c = 0; c < d; ++c) {
        double num = 0.0;
        for (int64_t a = 0; a < d; ++a) num += fq[a] * KV[a * d + c];
        O[i * d + c] = num / den;
      }
    }
    if (kv_out) memcpy(kv_out + h * d * d, KV, sizeof(double) * (size_t)(d * d));
    if (z_out) memcpy(z_out + h * d, z, sizeof(double) * (size_t)d);
  }
  free(KV);
  free(z);
  free(fq);
}

/* Quadratic order with an explicit n x n weight matrix W[i][j] = phi(Q_i).phi(K_j), each
 * row normalised by its sum, then multiplied by V ([G12] "Standard path" of the worked
 * example).  When causal != 0 only j <= i enter row i ([G12] "The recurrent view": S_t sums
 * over j <= t).  w_out ([BH][n][n], unnormalised W) may be NULL. */
void orc_quadratic(const double* q, const double* k, const double* v, double* out, int64_t BH,
                   int64_t n, int64_t d, int causal, int map, double* w_out) {
  double* W = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t h = 0; h < BH; ++h) {
    const double* Q = q + h * n * d;
    const double* K = k + h * n * d;
    const double* V = v + h * n * d;
    double* O = out + h * n * d;
    for (int64_t i = 0; i < n; ++i) {
      int64_t last = causal ? i : n - 1;
      double rowsum = 0.0;
      for (int64_t j = 0; j <= last; ++j) {
        double w = 0.0;
        for (int64_t a = 0; a < d; ++a) w += orc_phi(Q[i * d + a], map) * orc_phi(K[j * d + a], map);
        W[j] = w;
        rowsum += w;
        if (w_out) w_out[h * n * n + i * n + j] = w;
      }
      if (w_out)
        for (int64_t j = last + 1; j < n; ++j) w_out[h * n * n + i * n + j] = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j <= last; ++j) acc += (W[j] / rowsum) * V[j * d + c];
        O[i * d + c] = acc;
      }
    }
  }
  free(W);
}

/* Causal form as the recurrence of [G12] "The recurrent view": for t = 0..n-1,
 * S += phi(k_t) v_t^T, z += phi(k_t), out_t = phi(q_t)^T S / phi(q_t)^T z.
 * s0 ([BH][d][d]) and z0 ([BH][d]) give the state before token 0 (NULL: zero state);
 * s_fin / z_fin (may be NULL) receive the state after token n-1. */
void orc_causal_recurrent(const double* q, const double* k, const double* v, double* out,
                          int64_t BH, int64_t n, int64_t d, int map, const double* s0,
                          const double* z0, double* s_fin, double* z_fin) {
  double* S = (double*)malloc(sizeof(double) * (size_t)(d * d));
  double* z = (double*)malloc(sizeof(double) * (size_t)d);
  double* fk = (double*)malloc(sizeof(double) * (size_t)d);
  double* fq = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t h = 0; h < BH; ++h) {
    const double* Q = q + h * n * d;
    const double* K = k + h * n * d;
    const double* V = v + h * n * d;
    double* O = out + h * n * d;
    for (int64_t a = 0; a < d; ++a) {
      z[a] = z0 ? z0[h * d + a] : 0.0;
      for (int64_t c = 0; c < d; ++c) S[a * d + c] = s0 ? s0[h * d * d + a * d + c] : 0.0;
    }
    for (int64_t t = 0; t < n; ++t) {
      for (int64_t a = 0; a < d; ++a) fk[a] = orc_phi(K[t * d + a], map);
      for (int64_t a = 0; a < d; ++a) {
        z[a] += fk[a];
        for (int64_t c = 0; c < d; ++c) S[a * d + c] += fk[a] * V[t * d + c];
      }
      for (int64_t a = 0; a < d; ++a) fq[a] = orc_phi(Q[t * d + a], map);
      double den = 0.0;
      for (int64_t a = 0; a < d; ++a) den += fq[a] * z[a];
      for (int64_t c = 0; c < d; ++c) {
        double num = 0.0;
        for (int64_t a = 0; a < d; ++a) num += fq[a] * S[a * d + c];
        O[t * d + c] = num / den;
      }
    }
    if (s_fin) memcpy(s_fin + h * d * d, S, sizeof(double) * (size_t)(d * d));
    if (z_fin) memcpy(z_fin + h * d, z, sizeof(double) * (size_t)d);
  }
  free(S);
  free(z);
  free(fk);
  free(fq);
}

/* Causal form split into chunks of C tokens.  For the chunk [r0, r1) and a query i in it,
 * the keys j <= i split into j < r0, summarised by the state (S, z) carried from earlier
 * chunks, and r0 <= j <= i, taken pairwise as in the quadratic order.  After the chunk the
 * state absorbs all its tokens.  This is the recurrence above regrouped by associativity
 * ([G12] "Linear attention: reordering the matmuls" and "The recurrent view"); C = 1 is
 * the recurrence and C >= n is the masked quadratic order. */
void orc_causal_chunked(const double* q, const double* k, const double* v, double* out,
                        int64_t BH, int64_t n, int64_t d, int64_t C, int map) {
  double* S = (double*)malloc(sizeof(double) * (size_t)(d * d));
  double* z = (double*)malloc(sizeof(double) * (size_t)d);
  double* fq = (double*)malloc(sizeof(double) * (size_t)d);
  double* num = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t h = 0; h < BH; ++h) {
    const double* Q = q + h * n * d;
    const double* K = k + h * n * d;
    const double* V = v + h * n * d;
    double* O = out + h * n * d;
    for (int64_t a = 0; a < d; ++a) {
      z[a] = 0.0;
      for (int64_t c = 0; c < d; ++c) S[a * d + c] = 0.0;
    }
    for (int64_t r0 = 0; r0 < n; r0 += C) {
      int64_t r1 = r0 + C < n ? r0 + C : n;
      for (int64_t i = r0; i < r1; ++i) {
        for (int64_t a = 0; a < d; ++a) fq[a] = orc_phi(Q[i * d + a], map);
        /* inter-chunk part: phi(q_i)^T S and phi(q_i)^T z */
        double den = 0.0;
        for (int64_t a = 0; a < d; ++a) den += fq[a] * z[a];
        for (int64_t c = 0; c < d; ++c) {
          num[c] = 0.0;
          for (int64_t a = 0; a < d; ++a) num[c] += fq[a] * S[a * d + c];
        }
        /* intra-chunk part: masked pairwise weights for r0 <= j <= i */
        for (int64_t j = r0; j <= i; ++j) {
          double w = 0.0;
          for (int64_t a = 0; a < d; ++a) w += fq[a] * orc_phi(K[j * d + a], map);
          den += w;
          for (int64_t c = 0; c < d; ++c) num[c] += w * V[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c) O[i * d + c] = num[c] / den;
      }
      /* carry: fold the whole chunk into the state */
      for (int64_t j = r0; j < r1; ++j) {
        for (int64_t a = 0; a < d; ++a) {
          double fk = orc_phi(K[j * d + a], map);
          z[a] += fk;
          for (int64_t c = 0; c < d; ++c) S[a * d + c] += fk * V[j * d + c];
        }
      }
    }
  }
  free(S);
  free(z);
  free(fq);
  free(num);
}

/* One recurrent decode step for BH independent heads, in place on the state:
 * S += phi(k) v^T, z += phi(k), then out = phi(q)^T S / phi(q)^T z
 * ([G12] "The recurrent view"; A5: fixed-size state, O(1) memory per step).
 * q, k, v, out are [BH][d]; S is [BH][d][d]; z is [BH][d]. */
void orc_decode_step(const double* q, const double* k, const double* v, double* S, double* z,
                     double* out, int64_t BH, int64_t d, int map) {
  for (int64_t h = 0; h < BH; ++h) {
    double* Sh = S + h * d * d;
    double* zh = z + h * d;
    for (int64_t a = 0; a < d; ++a) {
      double fk = orc_phi(k[h * d + a], map);
      zh[a] += fk;
      for (int64_t c = 0; c < d; ++c) Sh[a * d + c] += fk * v[h * d + c];
    }
    double den = 0.0;
    for (int64_t a = 0; a < d; ++a) den += orc_phi(q[h * d + a], map) * zh[a];
    for (int64_t c = 0; c < d; ++c) {
      double num = 0.0;
      for (int64_t a = 0; a < d; ++a) num += orc_phi(q[h * d + a], map) * Sh[a * d + c];
      out[h * d + c] = num / den;
    }
  }
}

/* Selected output rows of ONE head by the quadratic definition, at O(n d) per row: for row
 * i, weights w_j = phi(Q_i).phi(K_j) over the keys j in keys(i) ({0..n-1}, or {0..i} when
 * causal), out_i = sum_j w_j V_j / sum_j w_j.  phik ([n][d]) holds phi(K) precomputed by
 * orc_phi_rows so that many rows can share it.  out_rows is [nrows][d]. */
void orc_rows(const double* q, const double* phik, const double* v, double* out_rows,
              int64_t n, int64_t d, const int64_t* rows, int64_t nrows, int causal, int map) {
  double* fq = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows[r];
    int64_t last = causal ? i : n - 1;
    for (int64_t a = 0; a < d; ++a) fq[a] = orc_phi(q[i * d + a], map);
    double den = 0.0;
    double* o = out_rows + r * d;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j <= last; ++j) {
      double w = 0.0;
      for (int64_t a = 0; a < d; ++a) w += fq[a] * phik[j * d + a];
      den += w;
      for (int64_t c = 0; c < d; ++c) o[c] += w * v[j * d + c];
    }
    for (int64_t c = 0; c < d; ++c) o[c] /= den;
  }
  free(fq);
}

/* phi applied elementwise to count values (helper for orc_rows). */
void orc_phi_rows(const double* x, double* y, int64_t count, int map) {
  for (int64_t i = 0; i < count; ++i) y[i] = orc_phi(x[i], map);
}

/* Aggregate state of a block of tokens for BH heads: S = sum_j phi(k_j) v_j^T and
 * z = sum_j phi(k_j) over the n tokens given ([G12] "The recurrent view"; the same sums
 * as KV and the key sum of the linear order).  k, v: [BH][n][d]; S: [BH][d][d]; z: [BH][d]
 * are ADDED to (so a caller can accumulate a state across blocks). */
void orc_state_accumulate(const double* k, const double* v, double* S, double* z, int64_t BH,
                          int64_t n, int64_t d, int map) {
  for (int64_t h = 0; h < BH; ++h) {
    const double* K = k + h * n * d;
    const double* V = v + h * n * d;
    for (int64_t j = 0; j < n; ++j) {
      for (int64_t a = 0; a < d; ++a) {
        double fk = orc_phi(K[j * d + a], map);
        z[h * d + a] += fk;
        for (int64_t c = 0; c < d; ++c) S[h * d * d + a * d + c] += fk * V[j * d + c];
      }
    }
  }
}
