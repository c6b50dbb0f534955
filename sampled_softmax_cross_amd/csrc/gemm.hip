// MFMA GEMMs of the step (gfx950, wave64):
//   logits  Z[T, P]   = x[T, d]  . W_C[P, d]^T   both operands k-contiguous
//   dX      dX[T, d]  = dZ[T, P] . W_C[P, d]     B is n-contiguous (k = P is its row index)
//   dW_C    dW_C[P,d] = dZ^T . x                 both operands m/n-contiguous (k = T),
//                                                split over k into fp32 slabs
// ("sampled_softmax.py", module docstring: the logits GEMM over C and the two
// gradient GEMMs are what the candidate set shrinks.)
//
// One kernel template serves all three. A 256-lane workgroup computes a BM x BN
// tile with 4 waves in a 2 x 2 grid; each wave issues v_mfma_f32_32x32x16_bf16
// (bf16) or eight v_mfma_f32_32x32x2f32 (fp32) per 16-wide k-step. Operand tiles
// live in LDS as rows of 128 bytes with k contiguous, double-buffered, with the
// 16-byte chunks of a row XOR-swizzled by the row index so that the fragment reads
// (32 rows x 16 bytes) and the transposing writes spread over the banks.
// An operand stored with k as its slow index is transposed in registers on its way
// to LDS (4 k-rows x one 16-byte vector per lane), so every MFMA reads k-contiguous
// fragments and no transposed copy of any operand is ever written to HBM.
#include "common.h"
#include "kernels.h"

namespace sce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;

// Index (in 16-byte units) of chunk `ch` of tile row `row`.
__device__ __forceinline__ int lds_index(int row, int ch) {
  return row * 8 + (ch ^ ((row ^ (row >> 3)) & 7));
}

template <typename TIn>
struct Elem {
  static constexpr int kSize = sizeof(TIn);
  static constexpr int kVec = 16 / kSize;   // elements per 16-byte vector
  static constexpr int kTileK = 128 / kSize; // k elements per LDS row
};

// Operand element (r, k) at P[r * ld + k]: 16-byte vectors along k.
template <typename TIn, int ROWS>
struct LoaderK {
  static constexpr int kVec = Elem<TIn>::kVec;
  static constexpr int kN = ROWS * 8 / kGemmThreads;
  static_assert(kN >= 1, "tile too small");
  uint4 r[kN];
  __device__ void load(const TIn* __restrict__ P, int64_t ld, int64_t r0, int64_t rlim, int64_t k0,
                       int64_t klim) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int v = threadIdx.x + kGemmThreads * i;
      const int64_t gr = r0 + (v >> 3);
      const int64_t gk = k0 + (v & 7) * kVec;
      r[i] = (gr < rlim && gk < klim) ? *reinterpret_cast<const uint4*>(P + gr * ld + gk)
                                      : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(uint4* __restrict__ tile) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int v = threadIdx.x + kGemmThreads * i;
      tile[lds_index(v >> 3, v & 7)] = r[i];
    }
  }
};

// Operand element (r, k) at P[k * ld + r]: each lane loads 4 k-rows of one 16-byte
// vector along r and writes them to LDS transposed (k contiguous).
template <typename TIn, int ROWS>
struct LoaderMN {
  static constexpr int kVec = Elem<TIn>::kVec;
  static constexpr int kChunks = ROWS / kVec;               // vectors across the tile
  static constexpr int kUnits = (Elem<TIn>::kTileK / 4) * kChunks;
  static constexpr int kN = kUnits / kGemmThreads;
  static_assert(kN >= 1 && kUnits % kGemmThreads == 0, "tile shape");
  uint4 r[kN][4];
  __device__ void load(const TIn* __restrict__ P, int64_t ld, int64_t r0, int64_t rlim, int64_t k0,
                       int64_t klim) {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int unit = threadIdx.x + kGemmThreads * u;
      const int64_t gr = r0 + (unit % kChunks) * kVec;
      const int64_t gk = k0 + (unit / kChunks) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        r[u][q] = (gr < rlim && gk + q < klim)
                      ? *reinterpret_cast<const uint4*>(P + (gk + q) * ld + gr)
                      : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(uint4* __restrict__ tile) const {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int unit = threadIdx.x + kGemmThreads * u;
      const int rc = unit % kChunks;
      const int kg = unit / kChunks;
      if constexpr (sizeof(TIn) == 2) {
        // 8 rows (tile rows rc*8+e), each gets 4 k-values = 8 bytes.
        const uint32_t* w0 = &r[u][0].x;
        const uint32_t* w1 = &r[u][1].x;
        const uint32_t* w2 = &r[u][2].x;
        const uint32_t* w3 = &r[u][3].x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t a0 = (w0[e >> 1] >> sh) & 0xffffu, a1 = (w1[e >> 1] >> sh) & 0xffffu;
          const uint32_t a2 = (w2[e >> 1] >> sh) & 0xffffu, a3 = (w3[e >> 1] >> sh) & 0xffffu;
          const int row = rc * 8 + e;
          uint2* dst = reinterpret_cast<uint2*>(tile + lds_index(row, kg >> 1)) + (kg & 1);
          *dst = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        }
      } else {
        // 4 rows (tile rows rc*4+e), each gets 4 k-values = 16 bytes.
        const uint32_t* w0 = &r[u][0].x;
        const uint32_t* w1 = &r[u][1].x;
        const uint32_t* w2 = &r[u][2].x;
        const uint32_t* w3 = &r[u][3].x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rc * 4 + e;
          tile[lds_index(row, kg)] = make_uint4(w0[e], w1[e], w2[e], w3[e]);
        }
      }
    }
  }
};

template <typename TIn, int ROWS, bool KC>
struct Loader;
template <typename TIn, int ROWS>
struct Loader<TIn, ROWS, true> : LoaderK<TIn, ROWS> {};
template <typename TIn, int ROWS>
struct Loader<TIn, ROWS, false> : LoaderMN<TIn, ROWS> {};

// Fragment of 8 consecutive k of one tile row for k-step `ks`.
template <typename TIn>
struct Frag;
template <>
struct Frag<bf16_t> {
  bf16x8_t v;
  __device__ void read(const uint4* tile, int row, int ks, int half) {
    const uint4 q = tile[lds_index(row, 2 * ks + half)];
    v = __builtin_bit_cast(bf16x8_t, q);
  }
};
template <>
struct Frag<float> {
  float v[8];
  __device__ void read(const uint4* tile, int row, int ks, int half) {
    const uint4 q0 = tile[lds_index(row, 4 * ks + 2 * half)];
    const uint4 q1 = tile[lds_index(row, 4 * ks + 2 * half + 1)];
    v[0] = __uint_as_float(q0.x); v[1] = __uint_as_float(q0.y);
    v[2] = __uint_as_float(q0.z); v[3] = __uint_as_float(q0.w);
    v[4] = __uint_as_float(q1.x); v[5] = __uint_as_float(q1.y);
    v[6] = __uint_as_float(q1.z); v[7] = __uint_as_float(q1.w);
  }
};

__device__ __forceinline__ void mma(f32x16_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
// fp32: lanes 0-31 supply k = q, lanes 32-63 supply k = 8 + q for the q-th
// 32x32x2 product, so eight products cover the 16 k of the step exactly once.
__device__ __forceinline__ void mma(f32x16_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int q = 0; q < 8; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[q], b.v[q], acc, 0, 0, 0);
}

enum OutMode { kOutBF16 = 0, kOutF32 = 1, kOutF32Split = 2 };

template <typename TIn, int BM, int BN, bool A_KC, bool B_KC, int OUT>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const TIn* __restrict__ A, int64_t lda,
                                                       const TIn* __restrict__ B, int64_t ldb,
                                                       void* __restrict__ Cout, int64_t ldc,
                                                       int64_t M, int64_t N, int64_t K,
                                                       int64_t kps, int64_t split_stride) {
  constexpr int TK = Elem<TIn>::kTileK;
  constexpr int KSTEPS = TK / 16;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ uint4 lds[2][(BM + BN) * 8];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t kb = (int64_t)blockIdx.z * kps;
  const int64_t ke = K < kb + kps ? K : kb + kps;
  const int nk = ke > kb ? (int)((ke - kb + TK - 1) / TK) : 0;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Loader<TIn, BM, A_KC> la;
  Loader<TIn, BN, B_KC> lb;
  if (nk > 0) {
    la.load(A, lda, m0, M, kb, ke);
    lb.load(B, ldb, n0, N, kb, ke);
    la.store(lds[0]);
    lb.store(lds[0] + BM * 8);
  }
  __syncthreads();
  const int arow = wm * WM + (lane & 31);
  const int brow = wn * WN + (lane & 31);
  const int half = lane >> 5;
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) {
      const int64_t k0 = kb + (int64_t)(it + 1) * TK;
      la.load(A, lda, m0, M, k0, ke);
      lb.load(B, ldb, n0, N, k0, ke);
    }
    const uint4* tA = lds[cur];
    const uint4* tB = lds[cur] + BM * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      Frag<TIn> fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i].read(tA, arow + i * 32, ks, half);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j].read(tB, brow + j * 32, ks, half);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    if (it + 1 < nk) {
      la.store(lds[cur ^ 1]);
      lb.store(lds[cur ^ 1] + BM * 8);
    }
    __syncthreads();
  }

  // Accumulator r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32 of
  // its 32 x 32 block.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < M && col < N) {
          if constexpr (OUT == kOutBF16) {
            static_cast<bf16_t*>(Cout)[row * ldc + col] = f32_to_bf16(acc[i][j][r]);
          } else if constexpr (OUT == kOutF32) {
            static_cast<float*>(Cout)[row * ldc + col] = acc[i][j][r];
          } else {
            static_cast<float*>(Cout)[(int64_t)blockIdx.z * split_stride + row * ldc + col] =
                acc[i][j][r];
          }
        }
      }
    }
}

int gemm_dw_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int s = 1;
  while (s < 16 && tiles * s < 512 && K / (2 * s) >= 1024) s *= 2;
  return s;
}

template <typename TIn, int BM, int BN, bool A_KC, bool B_KC, int OUT>
static hipError_t run(const GemmArgs& a, hipStream_t s) {
  constexpr int TK = Elem<TIn>::kTileK;
  const int splits = a.splits > 0 ? a.splits : 1;
  int64_t kps = (a.K + splits - 1) / splits;
  kps = (kps + TK - 1) / TK * TK;
  if (kps == 0) kps = TK;
  const int64_t gx = (a.N + BN - 1) / BN, gy = (a.M + BM - 1) / BM;
  if (gx == 0 || gy == 0) return hipGetLastError();
  if (gx > 0x7fffffff || gy > 65535 || splits > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm<TIn, BM, BN, A_KC, B_KC, OUT>), dim3((unsigned)gx, (unsigned)gy, splits),
                     dim3(kGemmThreads), 0, s, static_cast<const TIn*>(a.A), a.lda,
                     static_cast<const TIn*>(a.B), a.ldb, a.C, a.ldc, a.M, a.N, a.K, kps,
                     a.split_stride);
  return hipGetLastError();
}

hipError_t launch_gemm(Gemm kind, bool bf16, const GemmArgs& a, hipStream_t s) {
  if (bf16) {
    switch (kind) {
      case Gemm::Logits: return run<bf16_t, 128, 128, true, true, kOutBF16>(a, s);
      case Gemm::DX: return run<bf16_t, 128, 128, true, false, kOutBF16>(a, s);
      case Gemm::DW: return run<bf16_t, 128, 128, false, false, kOutF32Split>(a, s);
    }
  } else {
    switch (kind) {
      case Gemm::Logits: return run<float, 128, 128, true, true, kOutF32>(a, s);
      case Gemm::DX: return run<float, 128, 128, true, false, kOutF32>(a, s);
      case Gemm::DW: return run<float, 128, 128, false, false, kOutF32Split>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sce
