/*
 * Drives the C oracle (candidate build and loss/gradients) through its branches in a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_asan.py
 * compiles and runs it on the CPU). The oracle's sources are included as they are.
 * Prints "ok" and exits 0 when every call returned what it should and no sanitizer
 * report stopped the run.
 */
#include <stdio.h>

#include "../oracle/candidates.c"
#include "../oracle/ce.c"

static int fail(const char* what) {
  printf("FAIL %s\n", what);
  return 1;
}

/* C strictly ascending, |C| = P, every target a candidate at its position. */
static int check_set(int64_t V, int64_t P, int64_t T, const int64_t* y, const int32_t* C,
                     const int32_t* vpos, const int32_t* tpos) {
  for (int64_t j = 1; j < P; ++j)
    if (C[j] <= C[j - 1]) return 0;
  for (int64_t j = 0; j < P; ++j)
    if (C[j] < 0 || C[j] >= V || vpos[C[j]] != j) return 0;
  for (int64_t t = 0; t < T; ++t)
    if (y[t] >= 0 && (tpos[t] < 0 || C[tpos[t]] != y[t])) return 0;
  return 1;
}

int main(void) {
  enum { V = 4096, T = 1500, P = 2048, D = 8 };
  static int64_t y[T], p[T];
  static int32_t C[V], vpos[V], tpos[T], ppos[T];
  int64_t info[6];
  /* Labels: the first 1300 classes of the window (stride 1021, offset 0) force the
     fallback; the rest are no-ops or repeats. */
  for (int64_t t = 0; t < T; ++t) {
    y[t] = t < 1300 ? (t * 1021) % V : (t % 7 == 0 ? -1 : y[t % 1300]);
    p[t] = (t * 37) % V;
  }
  if (oracle_build_candidates(V, P, 1021, 0, T, y, p, C, vpos, tpos, ppos, info) != ORC_OK || !info[4])
    return fail("fallback build");
  if (!check_set(V, P, T, y, C, vpos, tpos)) return fail("fallback set");
  /* A window that wraps past the end of the sweep; P = V; the full softmax. */
  if (oracle_build_candidates(V, 300, 1021, V - 5, 40, y + 1400, NULL, C, vpos, tpos, NULL, info) != ORC_OK ||
      info[4] || !check_set(V, 300, 40, y + 1400, C, vpos, tpos))
    return fail("wrapping window");
  if (oracle_build_candidates(V, V, 3, 17, T, y, p, C, vpos, tpos, ppos, info) != ORC_OK ||
      !check_set(V, V, T, y, C, vpos, tpos))
    return fail("P = V");
  if (oracle_build_candidates(V, 0, 3, 17, T, y, p, NULL, vpos, tpos, ppos, info) != ORC_OK)
    return fail("P = 0");
  /* The conditions the page asserts, and labels out of range. */
  if (oracle_build_candidates(V, 100, 1021, 0, T, y, p, C, vpos, tpos, ppos, info) != ORC_TOO_MANY_TARGETS)
    return fail("too many targets");
  if (oracle_build_candidates(V, P, 2, 0, T, y, p, C, vpos, tpos, ppos, info) != ORC_BAD_ARG)
    return fail("stride not coprime");
  y[3] = V;
  if (oracle_build_candidates(V, P, 1021, 0, T, y, p, C, vpos, tpos, ppos, info) != ORC_TARGET_RANGE)
    return fail("label range");
  y[3] = -1;

  /* Loss and gradients over the fallback set on a small token slice. */
  if (oracle_build_candidates(V, P, 1021, 0, T, y, p, C, vpos, tpos, ppos, info) != ORC_OK)
    return fail("rebuild");
  enum { TS = 70 };
  static double x[TS * D], W[V * D], L[TS], rl[TS], out[2], dX[TS * D], dWC[P * D];
  for (int64_t i = 0; i < TS * D; ++i) x[i] = (double)((i * 7919) % 13) / 13.0 - 0.5;
  for (int64_t i = 0; i < V * D; ++i) W[i] = (double)((i * 104729) % 17) / 170.0 - 0.05;
  if (oracle_ce_lse(TS, D, P, x, W, C, NULL, TS, L) != CE_OK) return fail("lse");
  if (oracle_ce_loss(TS, D, P, x, W, C, L, tpos, ppos, rl, out) != CE_OK) return fail("loss");
  const int64_t N = (int64_t)out[1];
  if (oracle_ce_dx_rows(TS, D, P, x, W, C, L, tpos, ppos, N, NULL, TS, dX) != CE_OK) return fail("dx");
  if (oracle_ce_dwc_rows(TS, D, P, x, W, C, L, tpos, ppos, N, NULL, P, dWC) != CE_OK) return fail("dwc");
  /* sum_j g[t, j] = 0 for every row: the columns of dW_C sum to zero */
  for (int64_t k = 0; k < D; ++k) {
    double s = 0.0;
    for (int64_t j = 0; j < P; ++j) s += dWC[j * D + k];
    if (s > 1e-12 || s < -1e-12) return fail("dW_C columns sum to zero");
  }
  int64_t bad_rows[1] = {TS};
  if (oracle_ce_lse(TS, D, P, x, W, C, bad_rows, 1, L) != CE_BAD_ARG) return fail("row range");
  printf("ok\n");
  return 0;
}
