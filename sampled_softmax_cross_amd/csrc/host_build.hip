// The candidate build on the host ("sampled_softmax.py", CandidateBuilder: the page builds
// the set with numpy on a worker thread, with no device work, so that it stays off the
// training step's critical path, then uploads it).
//
// Same result as the device build (launch_candidates), computed with 64-bit bitmap
// words: marking sets bits, the distinct count is a popcount, the window walk tests bits
// in sweep order, the page's fallback counts free classes word by word, C is the set bits
// in ascending order, and a class's position is the count of set bits before its word plus
// those below it in the word. Everything lives on the stack (V <= SCE_MAX_V_SAMPLED: two
// arrays of 2048 words); nothing is allocated and nothing is shared between calls, so
// calls from different threads are independent.
#include <stdint.h>

#include "../../include/sampled_ce.h"

namespace {

constexpr int64_t kWords = SCE_MAX_V_SAMPLED / 64;

inline int popc(uint64_t w) { return __builtin_popcountll(w); }
inline bool has(const uint64_t* m, int64_t c) { return (m[c >> 6] >> (c & 63)) & 1u; }
inline void set(uint64_t* m, int64_t c) { m[c >> 6] |= 1ull << (c & 63); }
inline int64_t modv(int64_t a, int64_t m) {
  const int64_t r = a % m;
  return r < 0 ? r + m : r;
}
inline int64_t gcd(int64_t a, int64_t b) {
  while (b) {
    const int64_t r = a % b;
    a = b;
    b = r;
  }
  return a;
}

// Position of class c in C (-1 when c is not a candidate).
inline int32_t position(const uint64_t* m, const int32_t* before, int64_t c) {
  const uint64_t w = m[c >> 6];
  const int b = (int)(c & 63);
  if (!((w >> b) & 1u)) return -1;
  return before[c >> 6] + popc(w & ((1ull << b) - 1ull));
}

}  // namespace

extern "C" {

sce_status sce_build_candidates_host(const int64_t* targets, const int64_t* prefix_targets,
                                     int64_t T, int64_t V, int64_t P, int64_t stride,
                                     int64_t offset, int32_t* candidates_out,
                                     int32_t* target_pos_out, int32_t* prefix_pos_out,
                                     int64_t* aux_out) {
  if (T < 0 || V < 1 || V > SCE_MAX_V_SAMPLED || P < 1 || P > V) return SCE_EINVAL;
  if ((T > 0 && (targets == nullptr || target_pos_out == nullptr)) || candidates_out == nullptr)
    return SCE_EINVAL;
  const int64_t s = modv(stride, V);
  if (gcd(s, V) != 1) return SCE_EINVAL;
  const int64_t off = modv(offset, V);
  const int64_t nw = (V + 63) / 64;
  uint64_t mark[kWords];
  int32_t before[kWords];
  for (int64_t w = 0; w < nw; ++w) mark[w] = 0;

  // 1. targets (a label outside [-1, V) is flagged and dropped, like the device build)
  int status = 0;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t y = targets[t];
    if (y < -1 || y >= V) status |= SCE_DEV_LABEL_RANGE;
    else if (y >= 0) set(mark, y);
    if (prefix_targets != nullptr && (prefix_targets[t] < -1 || prefix_targets[t] >= V))
      status |= SCE_DEV_LABEL_RANGE;
  }
  int64_t distinct = 0;
  for (int64_t w = 0; w < nw; ++w) distinct += popc(mark[w]);

  int64_t next_off = off;
  if (distinct > P) {
    // the page asserts this never happens; flag it and take C = [0, P) (as the device does)
    status |= SCE_DEV_TOO_MANY_TARGETS;
    for (int64_t w = 0; w < nw; ++w) {
      const int64_t lo = w * 64;
      mark[w] = P >= lo + 64 ? ~0ull : (P > lo ? (1ull << (P - lo)) - 1ull : 0ull);
    }
  } else if (distinct < P) {
    const int64_t need = P - distinct;
    const int64_t draw = (17 * need) / 10 + 256 < V ? (17 * need) / 10 + 256 : V;
    next_off = (off + draw) % V;
    // 2. the window of the sweep, in sweep order; the picks go to a second bitmap so
    //    that the test stays against the targets alone
    uint64_t pick[kWords];
    for (int64_t w = 0; w < nw; ++w) pick[w] = 0;
    int64_t got = 0;
    int64_t c = (off * s) % V;
    for (int64_t i = 0; i < draw && got < need; ++i) {
      if (!has(mark, c)) {
        set(pick, c);
        ++got;
      }
      c += s;
      if (c >= V) c -= V;
    }
    if (got == need) {
      for (int64_t w = 0; w < nw; ++w) mark[w] |= pick[w];
    } else {
      // 3. the page's fallback: every step-th free class, ascending, the first `need`
      const int64_t step = (V - distinct) / need > 1 ? (V - distinct) / need : 1;
      int64_t rank = 0, taken = 0;
      for (int64_t w = 0; w < nw && taken < need; ++w) {
        const uint64_t valid = (w == nw - 1 && V % 64) ? (1ull << (V % 64)) - 1ull : ~0ull;
        uint64_t fm = ~mark[w] & valid;
        uint64_t sel = 0;
        while (fm && taken < need) {
          const int b = __builtin_ctzll(fm);
          fm &= fm - 1;
          if (rank % step == 0) {
            sel |= 1ull << b;
            ++taken;
          }
          ++rank;
        }
        mark[w] |= sel;
      }
    }
  }

  // 4. C ascending, and the set bits before each word
  int32_t n = 0;
  for (int64_t w = 0; w < nw; ++w) {
    before[w] = n;
    uint64_t m = mark[w];
    while (m) {
      candidates_out[n++] = (int32_t)(w * 64 + __builtin_ctzll(m));
      m &= m - 1;
    }
  }

  // 5. positions; N
  int64_t N = 0;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t y = targets[t];
    const int32_t tp = (y >= 0 && y < V) ? position(mark, before, y) : -1;
    target_pos_out[t] = tp;
    N += tp >= 0;
    const int64_t q = prefix_targets ? prefix_targets[t] : -1;
    const int32_t pp = (q >= 0 && q < V) ? position(mark, before, q) : -1;
    if (prefix_pos_out) prefix_pos_out[t] = pp;
    N += pp >= 0;
  }
  if (aux_out) {
    aux_out[0] = distinct;
    aux_out[1] = N;
    aux_out[2] = next_off;
    aux_out[3] = status;
  }
  return SCE_OK;
}

}  // extern "C"
