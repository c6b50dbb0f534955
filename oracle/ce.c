/*
 * Loss and gradient oracle in plain C, double precision, OpenMP over token blocks
 * (TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it; the HIP library never does, and nothing here is shared
 * with the HIP sources).
 *
 * What is computed, for one microbatch of T tokens (hidden states x [T, d]), the LM
 * head W [V, d] and a candidate set C of P classes (C == NULL: the whole vocabulary,
 * P = V), with label positions y'_t = tpos[t] and p'_t = ppos[t] (-1: no label):
 *   z[t, j] = sum_k x[t, k] W[C[j], k]
 *       ("sampled_softmax.py", module docstring: the logits are x times the candidate
 *       rows of the LM head, and labels are positions in C);
 *   L[t] = m[t] + ln sum_j exp(z[t, j] - m[t]),  m[t] = max_j z[t, j]
 *       ("Learning Triton one kernel at a time: softmax", softmax definition and the
 *       section on subtracting the row maximum);
 *   row_loss[t] = [y'_t >= 0](L[t] - z[t, y'_t]) + [p'_t >= 0](L[t] - z[t, p'_t]),
 *   N = number of labels with position >= 0, loss = sum_t row_loss[t] / N (0 if N = 0)
 *       ("16_optimization_checks.py", lm_gradient: summed token losses over the count
 *       of non-ignored targets);
 *   g[t, j] = (n_t exp(z[t, j] - L[t]) - [j = y'_t] - [j = p'_t]) / N, n_t the row's
 *       label count (the softmax-gradient section of the Triton article, applied to
 *       cross-entropy: softmax minus one-hot);
 *   dX[t, k] = sum_j g[t, j] W[C[j], k];   dW_C[j, k] = sum_t g[t, j] x[t, k].
 *
 * Every sum runs over its index in increasing order in double precision (the dot
 * products over k use the compiler's vector lanes, "omp simd", which only changes the
 * rounding order). The only restructuring is memory management: tokens (and, for
 * dW_C, candidate columns) are taken TB at a time so that the logits of a block are
 * held, never the whole [T, P]; each output element is still produced by the sum
 * above. Results do not depend on the number of threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { CE_OK = 0, CE_BAD_ARG = 1, CE_NO_MEMORY = 4 };

#define TB 64 /* tokens (or candidate columns) per block */

/* Threads an OpenMP region of this library uses (1 without OpenMP). */
int oracle_ce_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double dot(const double* a, const double* b, int64_t d) {
  double s = 0.0;
#pragma omp simd reduction(+ : s)
  for (int64_t k = 0; k < d; ++k) s += a[k] * b[k];
  return s;
}

static const double* cand_row(const double* W, const int32_t* C, int64_t j, int64_t d) {
  return W + (C ? (int64_t)C[j] : j) * d;
}

static int64_t row_of(const int64_t* rows, int64_t i) { return rows ? rows[i] : i; }

/* Logits z[i, j] = x[row_i] . W[C[j]] for the (at most TB) rows of one block. */
static void block_logits(const double* x, const double* W, const int32_t* C, int64_t d,
                         int64_t P, const int64_t* rows, int64_t r0, int64_t nb, double* z) {
  for (int64_t j = 0; j < P; ++j) {
    const double* w = cand_row(W, C, j, d);
    for (int64_t i = 0; i < nb; ++i) z[i * P + j] = dot(x + row_of(rows, r0 + i) * d, w, d);
  }
}

static double row_lse(const double* z, int64_t P) {
  double m = -INFINITY;
  for (int64_t j = 0; j < P; ++j) m = z[j] > m ? z[j] : m;
  double s = 0.0;
  for (int64_t j = 0; j < P; ++j) s += exp(z[j] - m);
  return m + log(s);
}

/* 1 when every index of idx[0..n) (all of [0, n) when idx == NULL) lies in [0, limit). */
static int in_range(const int64_t* idx, int64_t n, int64_t limit) {
  if (idx == NULL) return n <= limit;
  for (int64_t i = 0; i < n; ++i)
    if (idx[i] < 0 || idx[i] >= limit) return 0;
  return 1;
}

/* 1 when every label position is -1 or a candidate position. */
static int labels_ok(const int32_t* tpos, const int32_t* ppos, int64_t T, int64_t P) {
  for (int64_t t = 0; t < T; ++t) {
    if (tpos[t] < -1 || tpos[t] >= P) return 0;
    if (ppos != NULL && (ppos[t] < -1 || ppos[t] >= P)) return 0;
  }
  return 1;
}

static int64_t labels_of(const int32_t* tpos, const int32_t* ppos, int64_t t) {
  return (tpos[t] >= 0) + (ppos != NULL && ppos[t] >= 0);
}

/*
 * L[i] = log-sum-exp of the logits of row rows[i] (rows == NULL: row i), i < nrows.
 */
int oracle_ce_lse(int64_t T, int64_t d, int64_t P, const double* x, const double* W,
                  const int32_t* C, const int64_t* rows, int64_t nrows, double* L) {
  if (T < 0 || d <= 0 || P <= 0 || nrows < 0 || x == NULL || W == NULL || L == NULL ||
      !in_range(rows, nrows, T))
    return CE_BAD_ARG;
  const int64_t nblk = (nrows + TB - 1) / TB;
  int err = CE_OK;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * TB * (size_t)P);
    if (z == NULL) {
#pragma omp atomic write
      err = CE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      if (z == NULL) continue;
      const int64_t r0 = b * TB, nb = nrows - r0 < TB ? nrows - r0 : TB;
      block_logits(x, W, C, d, P, rows, r0, nb, z);
      for (int64_t i = 0; i < nb; ++i) L[r0 + i] = row_lse(z + i * P, P);
    }
    free(z);
  }
  return err;
}

/*
 * Given every row's L: row_loss [T], N and the loss (out[0] = loss, out[1] = N).
 * The label logits z[t, y'_t], z[t, p'_t] are single dot products.
 */
int oracle_ce_loss(int64_t T, int64_t d, int64_t P, const double* x, const double* W, const int32_t* C,
                   const double* L, const int32_t* tpos, const int32_t* ppos, double* row_loss,
                   double* out) {
  if (T < 0 || d <= 0 || (T > 0 && (x == NULL || L == NULL || tpos == NULL || row_loss == NULL)) ||
      W == NULL || out == NULL)
    return CE_BAD_ARG;
  if (!labels_ok(tpos, ppos, T, P)) return CE_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double l = 0.0;
    if (tpos[t] >= 0) l += L[t] - dot(x + t * d, cand_row(W, C, tpos[t], d), d);
    if (ppos != NULL && ppos[t] >= 0) l += L[t] - dot(x + t * d, cand_row(W, C, ppos[t], d), d);
    row_loss[t] = l;
  }
  int64_t N = 0;
  double sum = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    N += labels_of(tpos, ppos, t);
    sum += row_loss[t];
  }
  out[0] = N > 0 ? sum / (double)N : 0.0;
  out[1] = (double)N;
  return CE_OK;
}

/*
 * dX rows: dX[i, :] = sum_j g[rows[i], j] W[C[j], :] for i < nrows (rows == NULL: all),
 * from every row's L and N (all zero when N == 0).
 */
int oracle_ce_dx_rows(int64_t T, int64_t d, int64_t P, const double* x, const double* W,
                      const int32_t* C, const double* L, const int32_t* tpos,
                      const int32_t* ppos, int64_t N, const int64_t* rows, int64_t nrows,
                      double* dX) {
  if (T < 0 || d <= 0 || P <= 0 || nrows < 0 || x == NULL || W == NULL || dX == NULL ||
      (T > 0 && (L == NULL || tpos == NULL)) || !in_range(rows, nrows, T))
    return CE_BAD_ARG;
  if (!labels_ok(tpos, ppos, T, P)) return CE_BAD_ARG;
  memset(dX, 0, sizeof(double) * (size_t)nrows * (size_t)d);
  if (N == 0) return CE_OK;
  const int64_t nblk = (nrows + TB - 1) / TB;
  int err = CE_OK;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * TB * (size_t)P);
    if (z == NULL) {
#pragma omp atomic write
      err = CE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      if (z == NULL) continue;
      const int64_t r0 = b * TB, nb = nrows - r0 < TB ? nrows - r0 : TB;
      block_logits(x, W, C, d, P, rows, r0, nb, z);
      for (int64_t i = 0; i < nb; ++i) {
        const int64_t t = row_of(rows, r0 + i);
        const double n = (double)labels_of(tpos, ppos, t);
        double* out = dX + (r0 + i) * d;
        for (int64_t j = 0; j < P; ++j) {
          double g = n * exp(z[i * P + j] - L[t]);
          if (tpos[t] == j) g -= 1.0;
          if (ppos != NULL && ppos[t] == j) g -= 1.0;
          g /= (double)N;
          const double* w = cand_row(W, C, j, d);
#pragma omp simd
          for (int64_t k = 0; k < d; ++k) out[k] += g * w[k];
        }
      }
    }
    free(z);
  }
  return err;
}

/*
 * dW_C rows: out[i, :] = sum_t g[t, cols[i]] x[t, :] for i < ncols (cols == NULL: all P
 * candidate positions), over all T tokens, from every row's L and N.
 */
int oracle_ce_dwc_rows(int64_t T, int64_t d, int64_t P, const double* x, const double* W,
                       const int32_t* C, const double* L, const int32_t* tpos,
                       const int32_t* ppos, int64_t N, const int64_t* cols, int64_t ncols,
                       double* out) {
  if (T < 0 || d <= 0 || P <= 0 || ncols < 0 || W == NULL || out == NULL ||
      (T > 0 && (x == NULL || L == NULL || tpos == NULL)) || !in_range(cols, ncols, P))
    return CE_BAD_ARG;
  if (!labels_ok(tpos, ppos, T, P)) return CE_BAD_ARG;
  memset(out, 0, sizeof(double) * (size_t)ncols * (size_t)d);
  if (N == 0) return CE_OK;
  const int64_t nblk = (ncols + TB - 1) / TB;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nblk; ++b) {
    const int64_t c0 = b * TB, nb = ncols - c0 < TB ? ncols - c0 : TB;
    for (int64_t t = 0; t < T; ++t) {
      const double* xt = x + t * d;
      const double n = (double)labels_of(tpos, ppos, t);
      for (int64_t i = 0; i < nb; ++i) {
        const int64_t j = cols ? cols[c0 + i] : c0 + i;
        double g = n * exp(dot(xt, cand_row(W, C, j, d), d) - L[t]);
        if (tpos[t] == j) g -= 1.0;
        if (ppos != NULL && ppos[t] == j) g -= 1.0;
        g /= (double)N;
        double* o = out + (c0 + i) * d;
#pragma omp simd
        for (int64_t k = 0; k < d; ++k) o[k] += g * xt[k];
      }
    }
  }
  return CE_OK;
}
