// Fused row-wise cross-entropy forward + backward over the logits, in place.
//
// Per row t of Z [T, ldz] (P valid columns; columns [P, ldz) are padding):
//   L_t   = m_t + ln sum_j exp(Z_tj - m_t),  m_t = max_j Z_tj
//   loss_t = [y'>=0](L_t - Z_ty') + [p'>=0](L_t - Z_tp')
//   dZ_tj = (n_t exp(Z_tj - L_t) - [j=y'] - [j=p']) / N     (written over Z)
// ("Learning Triton one kernel at a time: softmax": max subtraction, the online
// softmax that merges running (max, sum) pairs, and the softmax gradient, here
// specialised to cross-entropy where the upstream gradient is a one-hot.)
//
// The row is read from HBM once into registers and written once: the kernel
// never re-reads Z and allocates no second [T, P] buffer. Each lane keeps its
// slice of the row as loaded and sweeps it twice (max and sum of exp(Z - m_lane),
// then exp(Z - L) for the gradient); lanes merge their (max, sum) pairs with the
// online-softmax rule (rescale the smaller-max sum by exp(m_small - m_big)). The
// rows' loss terms are summed by the last kernel of the step (the dense scatter).
#include "common.h"
#include "kernels.h"

namespace sce {

constexpr float kLog2e = 1.4426950408889634f;
// Rows whose lanes hold at most this many values keep exp(Z - m_lane) per element.
constexpr int kKeepValues = 40;
constexpr float kLn2 = 0.6931471805599453f;

template <typename TZ>
struct RowVec;  // 16 bytes of a row

template <>
struct RowVec<bf16_t> {
  static constexpr int kElems = 8;
  __device__ static void unpack(const uint4& q, float* f) {
    f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x); f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
    f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z); f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
  __device__ static float load1(const bf16_t* p) { return bf16_to_f32(*p); }
};

template <>
struct RowVec<float> {
  static constexpr int kElems = 4;
  __device__ static void unpack(const uint4& q, float* f) {
    f[0] = __uint_as_float(q.x); f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z); f[3] = __uint_as_float(q.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
  __device__ static float load1(const float* p) { return *p; }
};

// Row traffic is touched once: loads and stores stream past the caches (nontemporal).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream(uint4* p, const uint4& q) {
  const u32x4_t v = {q.x, q.y, q.z, q.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Merge two (max, sum) pairs of the online softmax; a max of -inf marks an empty pair.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f((m - M) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - M) * kLog2e);
  m = M;
}

// e4m3 output: 1 / s_g, where s_g is the smallest power of two with n_max / N <= 448 s_g,
// i.e. 2^-k for the largest k with n_max 2^k <= 448 N. Every |g| <= n_t / N <= n_max / N,
// so g / s_g stays within e4m3's largest finite value (448).
__device__ __forceinline__ float grad_inv_scale(int N, int n_max) {
  if (N <= 0) return 1.f;
  const unsigned long long q = 448ull * (unsigned)N / (unsigned)n_max;
  const int k = 63 - __clzll(q);
  return __int_as_float((127 + k) << 23);
}

// Row 0 completes the scale table once s_g is known.
__device__ __forceinline__ void write_grad_scales(const G8Out& go, float ginv) {
  const float sg = 1.0f / ginv;  // exact: a power of two
  go.scales[kScaleG] = sg;
  go.scales[kScaleDx] = sg * go.scales[kScaleW];
  go.scales[kScaleDw] = sg * go.scales[kScaleX];
  if (go.scales_out) go.scales_out[1] = sg;
}

// Eight gradient values (already divided by s_g) as e4m3 codes (round to nearest even).
__device__ __forceinline__ void store_g8(const G8Out& go, int t, int i, const float* g) {
  uint2 o;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(g[0], g[1], 0, false);
  o.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(g[2], g[3], w, true);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(g[4], g[5], 0, false);
  o.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(g[6], g[7], w, true);
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = {o.x, o.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(go.g8 + (int64_t)t * go.ldg + (int64_t)i * 8));
}

// Block-wide merge; every thread gets the row's (max, sum). Contains barriers.
template <int NT>
__device__ __forceinline__ void block_merge_ms(float& m, float& s, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave);
    const float s2 = __shfl_xor(s, o, kWave);
    merge_ms(m, s, m2, s2);
  }
  constexpr int NW = NT / kWave;
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[2 * wid] = m;
    red[2 * wid + 1] = s;
  }
  __syncthreads();
  float M = red[0], S = red[1];
#pragma unroll
  for (int w = 1; w < NW; ++w) merge_ms(M, S, red[2 * w], red[2 * w + 1]);
  m = M;
  s = S;
}

// Hides the packed row from the optimiser between sweeps, so that each sweep unpacks
// it again instead of keeping every unpacked value live (which would double the
// registers a row needs).
template <int VPT>
__device__ __forceinline__ void opaque(uint4 (&q)[VPT]) {
#pragma unroll
  for (int k = 0; k < VPT; ++k) asm volatile("" : "+v"(q[k].x), "+v"(q[k].y), "+v"(q[k].z), "+v"(q[k].w));
}

// Register-resident row: NT lanes x VPT vectors of 16 bytes cover the row. G8: the
// gradient goes out as e4m3 codes of g / s_g (go), Z is only read.
template <typename TZ, int NT, int VPT, bool G8>
__global__ __launch_bounds__(NT) void k_ce_rows(TZ* __restrict__ Z, int64_t ldz, int P,
                                                const int32_t* __restrict__ tpos,
                                                const int32_t* __restrict__ ppos,
                                                const int32_t* __restrict__ counters,
                                                float* __restrict__ row_loss,
                                                float* __restrict__ row_lse, G8Out go) {
  using RV = RowVec<TZ>;
  constexpr int E = RV::kElems;
  static_assert(!G8 || E == 8, "e4m3 output from bf16 rows");
  __shared__ float red[2 * (NT / kWave)];
  const int t = blockIdx.x;
  TZ* row = Z + (int64_t)t * ldz;
  uint4* rowv = reinterpret_cast<uint4*>(row);
  const int nvec = (int)(ldz / E);  // vectors in the padded row
  const int tp = tpos[t];
  const int pp = ppos[t];
  // The labels' logits, loaded by every lane from a clamped column: no branch, so no
  // wait before the row's own loads go out. The barrier of the row merge completes
  // them before any lane writes the gradient over the row.
  const float zt = RV::load1(row + (tp >= 0 ? tp : 0));
  const float zp = RV::load1(row + (pp >= 0 ? pp : 0));

  // The row stays in registers as loaded. Short rows (up to 40 values per lane) keep
  // exp(Z - m_lane) per element after the first sweep, so the gradient costs one
  // multiply (the kernel is close to ALU-bound there); long rows
  // keep only the packed 16-byte vectors (half the registers for bf16, so more rows
  // per CU keep loads in flight) and evaluate the exponential a second time.
  // Only the last vector of a row can hold padding columns (j >= P).
  constexpr bool kKeep = VPT * E <= kKeepValues;
  uint4 q[kKeep ? 1 : VPT];
  float v[kKeep ? VPT : 1][E];
  float m = -INFINITY;
  float s = 0.f;
  if constexpr (kKeep) {
    // Unpack at load (padding and vectors past the row become -inf), then replace each
    // value by exp(Z - m_lane). G8: every load is issued before the first use (a lane
    // past the row's last vector reads that vector again and discards it); a load inside
    // the branch below is followed there by a wait for that one load, so a lane's loads
    // go out one at a time. Measured on the same GPU: the e4m3-output CE at stage-0/1
    // 97.5 -> 80 us with the loads issued together, while the in-place CE (which writes
    // its gradient over the row it reads) ran 5% slower that way, so it keeps the loads
    // in its branch.
    uint4 raw[G8 ? VPT : 1];
    if constexpr (G8) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int i = threadIdx.x + k * NT;
        raw[k] = ld_stream(rowv + (i < nvec ? i : nvec - 1));
      }
      opaque(raw);  // keeps the compiler from sinking a load back into its branch
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < nvec) {
        if constexpr (G8) RV::unpack(raw[k], v[k]);
        else RV::unpack(ld_stream(rowv + i), v[k]);
        if ((i + 1) * E > P) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (i * E + e >= P) v[k][e] = -INFINITY;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[k][e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) m = fmaxf(m, v[k][e]);
    }
    const float mb = m == -INFINITY ? 0.f : m * kLog2e;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        v[k][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[k][e], kLog2e, -mb));  // exp2(-inf) = 0
        s += v[k][e];
      }
  } else {
    // Every load is issued before the first use: a lane past the row's last vector
    // reads that vector again (the sweeps below skip it). A load under a branch
    // would be followed, inside the branch, by a wait for that one load.
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = threadIdx.x + k * NT;
      q[k] = ld_stream(rowv + (i < nvec ? i : nvec - 1));
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < nvec) {
        float f[E];
        RV::unpack(q[k], f);
        const bool full = (i + 1) * E <= P;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (full || i * E + e < P) m = fmaxf(m, f[e]);
      }
    }
    const float mb = m == -INFINITY ? 0.f : m * kLog2e;
    opaque(q);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < nvec) {
        float f[E];
        RV::unpack(q[k], f);
        const bool full = (i + 1) * E <= P;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (full || i * E + e < P) s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], kLog2e, -mb));
      }
    }
  }
  float M = m, S = s;
  block_merge_ms<NT>(M, S, red);
  const float L = M + __builtin_amdgcn_logf(S) * kLn2;  // logf here is log2

  const int N = counters[kNumLabels];
  const float ginv = G8 ? grad_inv_scale(N, go.n_max) : 1.f;
  if constexpr (G8)
    if (t == 0 && threadIdx.x == 0) write_grad_scales(go, ginv);
  const float inv = N > 0 ? 1.0f / (float)N * ginv : 0.f;  // ginv: exact power of two
  const int nt = (tp >= 0) + (pp >= 0);
  // kKeep: exp(Z - L) = exp(Z - m_lane) * exp(m_lane - L); else exp(Z - L) directly.
  const float scale = kKeep ? (m == -INFINITY ? 0.f : (float)nt * inv * __builtin_amdgcn_exp2f((m - L) * kLog2e))
                            : (float)nt * inv;
  const float Lb = L * kLog2e;
  const int vt = tp >= 0 ? tp / E : -1;
  const int vp = pp >= 0 ? pp / E : -1;
  if constexpr (!kKeep) opaque(q);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < nvec) {
      float g[E];
      if constexpr (kKeep) {
#pragma unroll
        for (int e = 0; e < E; ++e) g[e] = v[k][e] * scale;  // 0 on padding columns
      } else {
        float f[E];
        RV::unpack(q[k], f);
        const bool full = (i + 1) * E <= P;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], kLog2e, -Lb)) * scale;
          g[e] = (full || i * E + e < P) ? x : 0.f;
        }
      }
      if (i == vt || i == vp) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = i * E + e;
          g[e] -= (float)((j == tp) + (j == pp)) * inv;
        }
      }
      if constexpr (G8) store_g8(go, t, i, g);
      else st_stream(rowv + i, RV::pack(g));
    }
  }
  if (threadIdx.x == 0) {
    float l = 0.f;
    if (tp >= 0) l += L - zt;
    if (pp >= 0) l += L - zp;
    row_loss[t] = l;
    if (row_lse) row_lse[t] = L;
  }
}

// Short rows (at most 64 * VPT vectors): one wave per row, four rows per workgroup,
// the (max, sum) merge by shuffles only (no LDS, no barrier). The same arithmetic as
// k_ce_rows with exp(Z - m_lane) kept per element.
template <typename TZ, int VPT, bool G8>
__global__ __launch_bounds__(256) void k_ce_rows_wave(TZ* __restrict__ Z, int64_t ldz, int P,
                                                      int T, const int32_t* __restrict__ tpos,
                                                      const int32_t* __restrict__ ppos,
                                                      const int32_t* __restrict__ counters,
                                                      float* __restrict__ row_loss,
                                                      float* __restrict__ row_lse, G8Out go) {
  using RV = RowVec<TZ>;
  constexpr int E = RV::kElems;
  static_assert(!G8 || E == 8, "e4m3 output from bf16 rows");
  const int lane = threadIdx.x & (kWave - 1);
  const int t = (int)blockIdx.x * 4 + (int)(threadIdx.x / kWave);
  if (t >= T) return;  // a whole wave
  TZ* row = Z + (int64_t)t * ldz;
  uint4* rowv = reinterpret_cast<uint4*>(row);
  const int nvec = (int)(ldz / E);
  // G8: every load issued before the first use, as in k_ce_rows (the row's vectors, then
  // the label logits from a clamped column: no branch, so no wait before they go out).
  // The in-place kernels keep the loads in their branches, as there.
  uint4 raw[G8 ? VPT : 1];
  if constexpr (G8) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = lane + k * kWave;
      raw[k] = ld_stream(rowv + (i < nvec ? i : nvec - 1));
    }
  }
  const int tp = tpos[t];
  const int pp = ppos[t];
  // the label logits (G8 writes the gradient to its own buffer, so the row is only read;
  // in place, they are read before any lane writes the row back)
  const float zt = G8 ? RV::load1(row + (tp >= 0 ? tp : 0)) : (tp >= 0 ? RV::load1(row + tp) : 0.f);
  const float zp = G8 ? RV::load1(row + (pp >= 0 ? pp : 0)) : (pp >= 0 ? RV::load1(row + pp) : 0.f);
  if constexpr (G8) opaque(raw);
  float v[VPT][E];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = lane + k * kWave;
    if (i < nvec) {
      if constexpr (G8) RV::unpack(raw[k], v[k]);
      else RV::unpack(ld_stream(rowv + i), v[k]);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (i * E + e >= P) v[k][e] = -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[k][e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) m = fmaxf(m, v[k][e]);
  }
  const float mb = m == -INFINITY ? 0.f : m * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      v[k][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[k][e], kLog2e, -mb));
      s += v[k][e];
    }
  float M = m, S = s;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(M, o, kWave);
    const float s2 = __shfl_xor(S, o, kWave);
    merge_ms(M, S, m2, s2);
  }
  const float L = M + __builtin_amdgcn_logf(S) * kLn2;  // logf here is log2
  const int N = counters[kNumLabels];
  const float ginv = G8 ? grad_inv_scale(N, go.n_max) : 1.f;
  if constexpr (G8)
    if (t == 0 && lane == 0) write_grad_scales(go, ginv);
  const float inv = N > 0 ? 1.0f / (float)N * ginv : 0.f;  // ginv: exact power of two
  const int nt = (tp >= 0) + (pp >= 0);
  const float scale = m == -INFINITY ? 0.f
                                     : (float)nt * inv * __builtin_amdgcn_exp2f((m - L) * kLog2e);
  const int vt = tp >= 0 ? tp / E : -1;
  const int vp = pp >= 0 ? pp / E : -1;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = lane + k * kWave;
    if (i < nvec) {
      float g[E];
#pragma unroll
      for (int e = 0; e < E; ++e) g[e] = v[k][e] * scale;
      if (i == vt || i == vp) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = i * E + e;
          g[e] -= (float)((j == tp) + (j == pp)) * inv;
        }
      }
      if constexpr (G8) store_g8(go, t, i, g);
      else st_stream(rowv + i, RV::pack(g));
    }
  }
  if (lane == 0) {
    float l = 0.f;
    if (tp >= 0) l += L - zt;
    if (pp >= 0) l += L - zp;
    row_loss[t] = l;
    if (row_lse) row_lse[t] = L;
  }
}

// Rows too long for registers: two sweeps over HBM (online (max, sum), then write).
template <typename TZ, int NT, bool G8>
__global__ __launch_bounds__(NT) void k_ce_rows_stream(TZ* __restrict__ Z, int64_t ldz, int P,
                                                       const int32_t* __restrict__ tpos,
                                                       const int32_t* __restrict__ ppos,
                                                       const int32_t* __restrict__ counters,
                                                       float* __restrict__ row_loss,
                                                       float* __restrict__ row_lse, G8Out go) {
  using RV = RowVec<TZ>;
  constexpr int E = RV::kElems;
  static_assert(!G8 || E == 8, "e4m3 output from bf16 rows");
  __shared__ float red[2 * (NT / kWave)];
  const int t = blockIdx.x;
  TZ* row = Z + (int64_t)t * ldz;
  uint4* rowv = reinterpret_cast<uint4*>(row);
  const int nvec = (int)(ldz / E);
  const int tp = tpos[t];
  const int pp = ppos[t];
  // the labels' logits: every lane, clamped column, no branch (as in k_ce_rows)
  const float zt = RV::load1(row + (tp >= 0 ? tp : 0));
  const float zp = RV::load1(row + (pp >= 0 ? pp : 0));
  float m = -INFINITY, s = 0.f;
  for (int i = threadIdx.x; i < nvec; i += NT) {
    float f[E];
    RV::unpack(ld_stream(rowv + i), f);
    float cm = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (i * E + e >= P) f[e] = -INFINITY;
      cm = fmaxf(cm, f[e]);
    }
    if (cm == -INFINITY) continue;
    float cs = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) cs += __builtin_amdgcn_exp2f((f[e] - cm) * kLog2e);
    merge_ms(m, s, cm, cs);
  }
  block_merge_ms<NT>(m, s, red);
  const float L = m + __builtin_amdgcn_logf(s) * kLn2;
  const int N = counters[kNumLabels];
  const float ginv = G8 ? grad_inv_scale(N, go.n_max) : 1.f;
  if constexpr (G8)
    if (t == 0 && threadIdx.x == 0) write_grad_scales(go, ginv);
  const float inv = N > 0 ? 1.0f / (float)N * ginv : 0.f;  // ginv: exact power of two
  const float c = (float)((tp >= 0) + (pp >= 0)) * inv;
  __syncthreads();  // every lane's label loads complete before any lane writes the row
  for (int i = threadIdx.x; i < nvec; i += NT) {
    float f[E];
    RV::unpack(ld_stream(rowv + i), f);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = i * E + e;
      f[e] = j < P ? c * __builtin_amdgcn_exp2f((f[e] - L) * kLog2e) -
                         (float)((j == tp) + (j == pp)) * inv
                   : 0.f;
    }
    if constexpr (G8) store_g8(go, t, i, f);
    else st_stream(rowv + i, RV::pack(f));
  }
  if (threadIdx.x == 0) {
    float l = 0.f;
    if (tp >= 0) l += L - zt;
    if (pp >= 0) l += L - zp;
    row_loss[t] = l;
    if (row_lse) row_lse[t] = L;
  }
}

template <typename TZ, int NT, int VPT, bool G8>
static void launch_ce_fixed(TZ* Z, int64_t ldz, int T, int P, const int32_t* tp, const int32_t* pp,
                            int32_t* counters, float* rl, float* lse, const G8Out& go, hipStream_t s) {
  hipLaunchKernelGGL((k_ce_rows<TZ, NT, VPT, G8>), dim3(T), dim3(NT), 0, s, Z, ldz, P, tp, pp,
                     counters, rl, lse, go);
}

template <typename TZ, int NT, bool G8>
static bool launch_ce_nt(int vpt, TZ* Z, int64_t ldz, int T, int P, const int32_t* tp,
                         const int32_t* pp, int32_t* counters, float* rl, float* lse,
                         const G8Out& go, hipStream_t s) {
  switch (vpt) {
#define SCE_CE_CASE(n) \
  case n:              \
    launch_ce_fixed<TZ, NT, n, G8>(Z, ldz, T, P, tp, pp, counters, rl, lse, go, s); \
    return true;
    SCE_CE_CASE(1) SCE_CE_CASE(2) SCE_CE_CASE(3) SCE_CE_CASE(4) SCE_CE_CASE(5) SCE_CE_CASE(6)
    SCE_CE_CASE(7) SCE_CE_CASE(8) SCE_CE_CASE(9) SCE_CE_CASE(10) SCE_CE_CASE(11) SCE_CE_CASE(12)
    SCE_CE_CASE(13) SCE_CE_CASE(14) SCE_CE_CASE(15) SCE_CE_CASE(16)
#undef SCE_CE_CASE
    default:
      return false;
  }
}

template <typename TZ, bool G8>
static void launch_ce_typed(TZ* Z, int64_t ldz, int T, int P, const int32_t* tp,
                            const int32_t* pp, int32_t* counters, float* rl, float* lse,
                            const G8Out& go, hipStream_t s) {
  constexpr int E = RowVec<TZ>::kElems;
  const int64_t nvec = ldz / E;
  if (nvec <= kWave * 4) {
    const int vpt = (int)((nvec + kWave - 1) / kWave);
    const dim3 grid((T + 3) / 4), block(256);
    if (vpt <= 1)
      hipLaunchKernelGGL((k_ce_rows_wave<TZ, 1, G8>), grid, block, 0, s, Z, ldz, P, T, tp, pp, counters, rl, lse, go);
    else if (vpt == 2)
      hipLaunchKernelGGL((k_ce_rows_wave<TZ, 2, G8>), grid, block, 0, s, Z, ldz, P, T, tp, pp, counters, rl, lse, go);
    else if (vpt == 3)
      hipLaunchKernelGGL((k_ce_rows_wave<TZ, 3, G8>), grid, block, 0, s, Z, ldz, P, T, tp, pp, counters, rl, lse, go);
    else
      hipLaunchKernelGGL((k_ce_rows_wave<TZ, 4, G8>), grid, block, 0, s, Z, ldz, P, T, tp, pp, counters, rl, lse, go);
  } else if (nvec <= 256 * kKeepValues / E) {
    // 256 lanes while they hold at most kKeepValues values each (exp(Z - m_lane) kept,
    // not evaluated twice), then 512 lanes, kept while that fits (P = 14336 bf16: 512 x 4
    // kept ran the CE 7.5% faster than 256 x 7 evaluated twice) and with more vectors
    // per lane past it (P = 24576 bf16: 512 x 6 at 70 registers ran 16% faster than
    // 256 x 12 at 99, and 1024 x 3 kept 45% slower).
    launch_ce_nt<TZ, 256, G8>((int)((nvec + 255) / 256), Z, ldz, T, P, tp, pp, counters, rl, lse,
                              go, s);
  } else if (nvec <= 512 * 16) {
    launch_ce_nt<TZ, 512, G8>((int)((nvec + 511) / 512), Z, ldz, T, P, tp, pp, counters, rl, lse,
                              go, s);
  } else {
    hipLaunchKernelGGL((k_ce_rows_stream<TZ, 1024, G8>), dim3(T), dim3(1024), 0, s, Z, ldz, P, tp,
                       pp, counters, rl, lse, go);
  }
}

// Label positions given by a caller (the CE alone): one workgroup copies them with
// every position outside [-1, P) replaced by -1 (flagged), counts N and sets the
// counters the CE kernel and the loss reduction read.
__global__ __launch_bounds__(1024) void k_ce_prep(const int32_t* __restrict__ tpos_in,
                                                  const int32_t* __restrict__ ppos_in, int T,
                                                  int P, int32_t* __restrict__ tpos,
                                                  int32_t* __restrict__ ppos,
                                                  int32_t* __restrict__ counters) {
  __shared__ int scratch[1024 / kWave + 1];
  int n = 0, bad = 0;
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    int a = tpos_in[t];
    if (a < -1 || a >= P) {
      bad = 1;
      a = -1;
    }
    tpos[t] = a;
    n += a >= 0;
    int b = ppos_in ? ppos_in[t] : -1;
    if (b < -1 || b >= P) {
      bad = 1;
      b = -1;
    }
    ppos[t] = b;
    n += b >= 0;
  }
  const int N = block_sum_int(n, scratch);
  const int any_bad = block_sum_int(bad, scratch);
  if (threadIdx.x == 0) {
    for (int i = 0; i < kNumCounters; ++i) counters[i] = 0;
    counters[kNumLabels] = N;
    counters[kStatus] = any_bad ? kDevLabelRange : 0;
  }
}

hipError_t launch_ce_prep(const int32_t* tpos_in, const int32_t* ppos_in, int T, int P,
                          int32_t* tpos, int32_t* ppos, int32_t* counters, hipStream_t s) {
  hipLaunchKernelGGL(k_ce_prep, dim3(1), dim3(1024), 0, s, tpos_in, ppos_in, T, P, tpos, ppos,
                     counters);
  return hipGetLastError();
}

hipError_t launch_ce_rows(void* Z, int64_t ldz, int T, int P, bool bf16,
                          const int32_t* target_pos, const int32_t* prefix_pos,
                          const int32_t* counters, float* row_loss, float* row_lse,
                          hipStream_t s) {
  if (T <= 0) return hipGetLastError();
  const G8Out none{};
  if (bf16)
    launch_ce_typed<bf16_t, false>(static_cast<bf16_t*>(Z), ldz, T, P, target_pos, prefix_pos,
                                   const_cast<int32_t*>(counters), row_loss, row_lse, none, s);
  else
    launch_ce_typed<float, false>(static_cast<float*>(Z), ldz, T, P, target_pos, prefix_pos,
                                  const_cast<int32_t*>(counters), row_loss, row_lse, none, s);
  return hipGetLastError();
}

hipError_t launch_ce_rows_g8(const void* Z, int64_t ldz, int T, int P, const int32_t* target_pos,
                             const int32_t* prefix_pos, const int32_t* counters, float* row_loss,
                             float* row_lse, const G8Out& go, hipStream_t s) {
  // the kernels write the codes of columns [0, ldz) (zeros past P) in rows ldg apart; a
  // wider pitch would leave bytes the e4m3 products read unwritten
  if (go.ldg != ldz || ldz % 16 != 0) return hipErrorInvalidValue;
  if (T <= 0) return hipGetLastError();
  launch_ce_typed<bf16_t, true>(static_cast<bf16_t*>(const_cast<void*>(Z)), ldz, T, P, target_pos,
                                prefix_pos, const_cast<int32_t*>(counters), row_loss, row_lse, go, s);
  return hipGetLastError();
}

}  // namespace sce
