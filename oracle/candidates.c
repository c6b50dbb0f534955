/*
 * Candidate-set oracle (TEST INFRASTRUCTURE ONLY).
 *
 * A plain, sequential, obviously-correct C version of the candidate build that
 * the sampled-softmax training loss runs once per microbatch. It exists to check
 * the GPU path and is never called by it: only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark load this file's library. It shares
 * no code, header or constant with the HIP sources.
 *
 * Source: "sampled_softmax.py" (modded-nanogpt, track_1_short course mirror):
 *   - module docstring: C is the set of distinct labels of the microbatch topped
 *     up with filler classes from a window of the cyclic order k*stride mod V (a
 *     permutation since gcd(stride, V) = 1); prefix labels only look classes up
 *     in C (position -1 when absent) and never add one;
 *   - CandidateBuilder.__init__ / reset: the sweep and its offset into it;
 *   - CandidateBuilder._negatives: window length, window advance, the fallback;
 *   - CandidateBuilder.build: marking, the distinct-count check, ascending C,
 *     and the class -> position map used for targets and prefix targets.
 *
 * Everything is int64 and strictly sequential; nothing is blocked or reordered.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
  ORC_OK = 0,
  ORC_BAD_ARG = 1,          /* V<=0, P<0, P>V, T<0, gcd(stride, V) != 1, null pointer */
  ORC_TOO_MANY_TARGETS = 2, /* more distinct targets than P (the page asserts)          */
  ORC_TARGET_RANGE = 3,     /* a target or prefix target outside [-1, V)                */
  ORC_NO_MEMORY = 4
};

static int64_t gcd_i64(int64_t a, int64_t b) {
  if (a < 0) a = -a;
  if (b < 0) b = -b;
  while (b != 0) {
    int64_t r = a % b;
    a = b;
    b = r;
  }
  return a;
}

static int64_t mod_i64(int64_t a, int64_t m) {
  int64_t r = a % m;
  return r < 0 ? r + m : r;
}

/*
 * info[0] = number of distinct targets (classes marked by targets alone)
 * info[1] = need   (P - distinct; 0 when no negatives are drawn)
 * info[2] = draw   (window length; 0 when need == 0)
 * info[3] = next_offset (the sweep offset after this candidate set is drawn)
 * info[4] = 1 if the fallback (every s-th free class) supplied the negatives
 * info[5] = N, the number of labels that survive the remap (target and prefix
 *           positions that are >= 0)
 *
 * P == 0 is the full softmax: no candidate set is built, C is [0, V) and every
 * position is the class id itself; offset is returned unchanged (reduced mod V).
 */
int oracle_build_candidates(int64_t V, int64_t P, int64_t stride, int64_t offset, int64_t T,
                            const int64_t* targets, const int64_t* prefix_targets,
                            int32_t* C, int32_t* vocab_pos, int32_t* target_pos,
                            int32_t* prefix_pos, int64_t* info) {
  if (V <= 0 || P < 0 || P > V || T < 0 || info == NULL || vocab_pos == NULL) return ORC_BAD_ARG;
  if (T > 0 && (targets == NULL || target_pos == NULL)) return ORC_BAD_ARG;
  if (prefix_targets != NULL && T > 0 && prefix_pos == NULL) return ORC_BAD_ARG;
  if (P > 0 && C == NULL) return ORC_BAD_ARG;
  int64_t s = mod_i64(stride, V);
  if (gcd_i64(s, V) != 1) return ORC_BAD_ARG;
  int64_t off = mod_i64(offset, V);
  for (int k = 0; k < 6; ++k) info[k] = 0;

  /* Range check first: -1 is the no-op label, anything else must be a class. */
  for (int64_t t = 0; t < T; ++t) {
    if (targets[t] < -1 || targets[t] >= V) return ORC_TARGET_RANGE;
    if (prefix_targets != NULL && (prefix_targets[t] < -1 || prefix_targets[t] >= V))
      return ORC_TARGET_RANGE;
  }

  /* One mark per class that occurs as a label (a target) in this microbatch. */
  unsigned char* mark = (unsigned char*)calloc((size_t)V, 1);
  if (mark == NULL) return ORC_NO_MEMORY;
  for (int64_t t = 0; t < T; ++t)
    if (targets[t] >= 0) mark[targets[t]] = 1;
  int64_t distinct = 0;
  for (int64_t c = 0; c < V; ++c) distinct += mark[c];
  info[0] = distinct;

  if (P == 0) {
    /* Full softmax: the vocabulary itself is the candidate set. */
    for (int64_t c = 0; c < V; ++c) vocab_pos[c] = (int32_t)c;
    info[3] = off;
  } else {
    if (distinct > P) {
      free(mark);
      return ORC_TOO_MANY_TARGETS;
    }
    int64_t need = P - distinct;
    info[1] = need;
    info[3] = off;
    if (need > 0) {
      /* Window length: 1.7 times what is needed plus 256, never more than V.
         Computed the way the page does, in double precision then truncated. */
      int64_t draw = (int64_t)((double)need * 1.7) + 256;
      if (draw > V) draw = V;
      info[2] = draw;

      /* Walk the window in sweep order; keep the classes that are not yet marked.
         Sweep entry k is (stride * k) mod V for k in [0, V); a window that runs
         past the end of the sweep continues at its start. */
      int64_t* kept = (int64_t*)malloc(sizeof(int64_t) * (size_t)draw);
      if (kept == NULL) {
        free(mark);
        return ORC_NO_MEMORY;
      }
      int64_t nkept = 0;
      for (int64_t i = 0; i < draw; ++i) {
        int64_t k = (off + i) % V;
        int64_t cls = (k * s) % V;
        if (!mark[cls]) kept[nkept++] = cls;
      }
      info[3] = (off + draw) % V;

      if (nkept >= need) {
        /* The first `need` unmarked classes of the window become negatives. */
        for (int64_t i = 0; i < need; ++i) mark[kept[i]] = 1;
      } else {
        /* Fallback: the window is discarded; take every step-th free class in
           ascending order, step = max(1, free_count div need), first `need`. */
        info[4] = 1;
        int64_t nfree = V - distinct; /* >= need because P <= V */
        int64_t step = nfree / need;
        if (step < 1) step = 1;
        int64_t rank = 0, taken = 0;
        unsigned char* chosen = (unsigned char*)calloc((size_t)V, 1);
        if (chosen == NULL) {
          free(kept);
          free(mark);
          return ORC_NO_MEMORY;
        }
        for (int64_t c = 0; c < V && taken < need; ++c) {
          if (mark[c]) continue;
          if (rank % step == 0) {
            chosen[c] = 1;
            ++taken;
          }
          ++rank;
        }
        for (int64_t c = 0; c < V; ++c)
          if (chosen[c]) mark[c] = 1;
        free(chosen);
      }
      free(kept);
    }

    /* C in ascending class order, and the inverse map class -> position. */
    int64_t n = 0;
    for (int64_t c = 0; c < V; ++c) {
      if (mark[c]) {
        C[n] = (int32_t)c;
        vocab_pos[c] = (int32_t)n;
        ++n;
      } else {
        vocab_pos[c] = -1;
      }
    }
    if (n != P) { /* cannot happen: distinct + need == P */
      free(mark);
      return ORC_BAD_ARG;
    }
  }
  free(mark);

  /* Remap labels to positions; -1 (no label) stays -1, and a prefix target that
     is not a candidate becomes -1 as well. */
  int64_t N = 0;
  for (int64_t t = 0; t < T; ++t) {
    target_pos[t] = targets[t] < 0 ? -1 : vocab_pos[targets[t]];
    if (target_pos[t] >= 0) ++N;
    if (prefix_targets != NULL) {
      prefix_pos[t] = prefix_targets[t] < 0 ? -1 : vocab_pos[prefix_targets[t]];
      if (prefix_pos[t] >= 0) ++N;
    } else if (prefix_pos != NULL) {
      prefix_pos[t] = -1;
    }
  }
  info[5] = N;
  return ORC_OK;
}
