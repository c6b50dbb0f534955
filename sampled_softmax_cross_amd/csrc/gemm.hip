// MFMA GEMMs of the step (gfx950, wave64):
//   logits  Z[T, P]   = x[T, d]  . W_C[P, d]^T   both operands k-contiguous
//   dX      dX[T, d]  = dZ[T, P] . W_C[P, d]     B is n-contiguous (k = P is its row index)
//   dW_C    dW_C[P,d] = dZ^T . x                 both operands m/n-contiguous (k = T),
//                                                split over k into fp32 slabs
// ("sampled_softmax.py", module docstring: the logits GEMM over C and the two
// gradient GEMMs are what the candidate set shrinks.)
//
// One kernel template serves all three. A 256-lane workgroup computes a BM x BN
// tile with 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2) block of
// fp32 accumulators (up to 128 x 128, i.e. 16 v_mfma_f32_32x32x16_bf16 per 16-wide
// k-step), which is what keeps the LDS fragment traffic below the LDS bandwidth:
// a wave reads (BM/2 + BN/2) x 32 bytes of fragments per k-step for
// (BM/2)(BN/2)/1024 MFMAs. fp32 inputs use eight v_mfma_f32_32x32x2f32 per k-step.
//
// Operand tiles live in LDS as rows of 128 bytes (k contiguous), double-buffered,
// with the 16-byte chunks of a row XOR-swizzled by the row index so fragment reads
// (32 rows x 16 bytes per half-wave) and tile writes spread over all banks. An
// operand stored with k as its slow index is transposed in registers on its way to
// LDS (4 k-rows of one 16-byte vector per lane), so every MFMA reads k-contiguous
// fragments and no transposed copy of any operand is written to HBM.
//
// Workgroups are renumbered so that each of the 8 XCDs (which receive workgroup ids
// round-robin) works on a contiguous, grouped block of output tiles whose operand
// panels then stay in that XCD's L2. bf16 results are staged through LDS so every
// lane stores whole 16-byte vectors of consecutive columns.
#include "gemm_common.h"

namespace sce {

// Operand element (r, k) at P[r * ld + k], loaded straight into LDS (buffer_load
// ... lds): instruction i of wave w fills the 64 consecutive 16-byte LDS chunks of
// tile rows 8b .. 8b+7 (b = w * kN + i), lane L the chunk 8b*8 + L. The lane picks
// the global chunk whose swizzled position that is, so the tile lands in LDS in the
// same layout the fragment reads expect, with no VGPR staging and no ds_write.
template <typename TIn, int ROWS>
struct LoaderK {
  static constexpr int kVec = Elem<TIn>::kVec;
  static constexpr int kN = ROWS * 8 / kGemmThreads;  // instructions per wave
  static_assert(kN >= 1 && (ROWS * 8) % kGemmThreads == 0, "tile shape");
  int off[kN];  // byte offset in the tile, or kOOB for rows outside the matrix
  int kch[kN];  // k offset (elements) of the lane's chunk
  int blk0;     // first 8-row block of this wave
  __device__ __forceinline__ void init(int64_t ld, int64_t rows_valid) {
    const int lane = threadIdx.x & 63;
    blk0 = (threadIdx.x >> 6) * kN;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int b = blk0 + i;
      const int row = 8 * b + (lane >> 3);
      const int ch = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
      kch[i] = ch * kVec;
      off[i] = row < rows_valid ? (int)((row * ld + kch[i]) * (int64_t)sizeof(TIn)) : kOOB;
    }
  }
  // base: address of tile element (0, 0); k_valid clips the tile along k.
  __device__ __forceinline__ void load(const TIn* base, int64_t k_valid, uint4* tile) const {
    const rsrc_t rs = make_rsrc(base);
#pragma unroll
    for (int i = 0; i < kN; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + (blk0 + i) * 64), 16,
          kch[i] < k_valid ? off[i] : kOOB, 0, 0, 0);
  }
  __device__ __forceinline__ void store(uint4*) const {}
};

// Operand element (r, k) at P[k * ld + r]: each lane loads 4 k-rows of one 16-byte
// vector along r and writes them to LDS transposed (k contiguous).
template <typename TIn, int ROWS>
struct LoaderMN {
  static constexpr int kVec = Elem<TIn>::kVec;
  static constexpr int kChunks = ROWS / kVec;  // vectors across the tile
  static constexpr int kUnits = (Elem<TIn>::kTileK / 4) * kChunks;
  static constexpr int kN = (kUnits + kGemmThreads - 1) / kGemmThreads;
  uint4 r[kN][4];
  int ldb;         // bytes between k-rows
  int rows_valid;  // tile rows inside the matrix
  __device__ __forceinline__ void init(int64_t ld, int64_t rows) {
    ldb = (int)(ld * (int64_t)sizeof(TIn));
    rows_valid = rows < ROWS ? (int)rows : ROWS;
  }
  __device__ __forceinline__ void load(const TIn* base, int64_t k_valid, uint4*) {
    const rsrc_t rs = make_rsrc(base);
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int unit = threadIdx.x + kGemmThreads * u;
      const int rc = unit % kChunks, kg = unit / kChunks;
      const bool ok = (kUnits % kGemmThreads == 0 || unit < kUnits) && rc * kVec < rows_valid;
      const int o = kg * 4 * ldb + rc * 16;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        r[u][q] = bload(rs, ok && kg * 4 + q < k_valid ? o + q * ldb : kOOB);
    }
  }
  __device__ __forceinline__ void store(uint4* __restrict__ tile) const {
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      const int unit = threadIdx.x + kGemmThreads * u;
      if (kUnits % kGemmThreads != 0 && unit >= kUnits) continue;
      const int rc = unit % kChunks;
      const int kg = unit / kChunks;
      const uint32_t* w0 = &r[u][0].x;
      const uint32_t* w1 = &r[u][1].x;
      const uint32_t* w2 = &r[u][2].x;
      const uint32_t* w3 = &r[u][3].x;
      if constexpr (sizeof(TIn) == 2) {
        // 8 tile rows (rc*8 + e) each receive 4 k-values = 8 bytes.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t a0 = (w0[e >> 1] >> sh) & 0xffffu, a1 = (w1[e >> 1] >> sh) & 0xffffu;
          const uint32_t a2 = (w2[e >> 1] >> sh) & 0xffffu, a3 = (w3[e >> 1] >> sh) & 0xffffu;
          uint2* dst = reinterpret_cast<uint2*>(tile + lds_index(rc * 8 + e, kg >> 1)) + (kg & 1);
          *dst = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        }
      } else {
        // 4 tile rows (rc*4 + e) each receive 4 k-values = 16 bytes.
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tile[lds_index(rc * 4 + e, kg)] = make_uint4(w0[e], w1[e], w2[e], w3[e]);
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

// Fragment: 8 consecutive k of one tile row for k-step `ks` (half = lane / 32).
template <typename TIn>
struct Frag;
template <>
struct Frag<bf16_t> {
  bf16x8_t v;
  __device__ __forceinline__ void read(const uint4* tile, int row, int ks, int half) {
    v = __builtin_bit_cast(bf16x8_t, tile[lds_index(row, 2 * ks + half)]);
  }
};
template <>
struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void read(const uint4* tile, int row, int ks, int half) {
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

template <typename TIn, int BM, int BN, bool A_KC, bool B_KC, int OUT>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(
    const TIn* __restrict__ A, int64_t lda, const TIn* __restrict__ B, int64_t ldb,
    void* __restrict__ Cout, int64_t ldc, int64_t M, int64_t N, int64_t K, int64_t kps,
    int64_t split_stride) {
  constexpr int TK = Elem<TIn>::kTileK;
  constexpr int KSTEPS = TK / 16;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = (BM + BN) * 8;  // uint4 per LDS stage
  __shared__ uint4 lds[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int nbx = (int)((N + BN - 1) / BN), nby = (int)((M + BM - 1) / BM);
  int tm, tn;
  tile_of(blockIdx.x, nby, nbx, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t kb = (int64_t)blockIdx.y * kps;
  const int64_t ke = K < kb + kps ? K : kb + kps;
  const int nk = ke > kb ? (int)((ke - kb + TK - 1) / TK) : 0;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Element (r, k) of an operand: r * ld + k (k-contiguous) or k * ld + r.
  auto tile_base = [](const TIn* P, int64_t ld, bool kc, int64_t r0, int64_t k0) {
    return kc ? P + r0 * ld + k0 : P + k0 * ld + r0;
  };
  Loader<TIn, BM, A_KC> la;
  Loader<TIn, BN, B_KC> lb;
  la.init(lda, M - m0);
  lb.init(ldb, N - n0);
  if (nk > 0) {
    la.load(tile_base(A, lda, A_KC, m0, kb), ke - kb, lds);
    lb.load(tile_base(B, ldb, B_KC, n0, kb), ke - kb, lds + BM * 8);
    la.store(lds);
    lb.store(lds + BM * 8);
  }
  vm_wait_all();
  __syncthreads();
  const int arow = wm * WM + (lane & 31);
  const int brow = wn * WN + (lane & 31);
  const int half = lane >> 5;
  // Fragments are double-buffered across k-steps: the reads for step s + 1 are in
  // flight while the MFMAs of step s run, so LDS latency stays off the MFMA path.
  Frag<TIn> fa[2][TM], fb[2][TN];
  auto read_frags = [&](const uint4* stage, int ks, int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i].read(stage, arow + i * 32, ks, half);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j].read(stage + BM * 8, brow + j * 32, ks, half);
  };
  if (nk > 0) read_frags(lds, 0, 0);
  for (int it = 0; it < nk; ++it) {
    const uint4* cur = lds + (it & 1) * STAGE;
    uint4* nxt = lds + ((it + 1) & 1) * STAGE;
    const bool more = it + 1 < nk;
    if (more) {
      const int64_t k0 = kb + (int64_t)(it + 1) * TK;
      la.load(tile_base(A, lda, A_KC, m0, k0), ke - k0, nxt);
      lb.load(tile_base(B, ldb, B_KC, n0, k0), ke - k0, nxt + BM * 8);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int c = ks & 1;  // KSTEPS is even: step 0 of every tile uses buffer 0
      if (ks + 1 < KSTEPS) read_frags(cur, ks + 1, c ^ 1);
      // The B-tile fragment is the MFMA's first operand, so each accumulator block
      // is the transposed 32 x 32 output: lane l holds output row (l % 32) and four
      // consecutive output columns per group of four registers.
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma(acc[i][j], fb[c][j], fa[c][i]);
      if (ks + 1 < KSTEPS) {
        // Issue order: one MFMA, one fragment read, ... then the remaining MFMAs.
        constexpr int kReads = (TM + TN) * (sizeof(TIn) == 2 ? 1 : 2);
        constexpr int kMfma = TM * TN * (sizeof(TIn) == 2 ? 1 : 8);
        static_assert(kMfma >= kReads, "schedule");
#pragma unroll
        for (int g = 0; g < kReads; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
      }
    }
    if (more) {
      la.store(nxt);
      lb.store(nxt + BM * 8);
    }
    vm_wait_all();  // direct-to-LDS loads of the next tile have landed
    __syncthreads();
    if (more) read_frags(nxt, 0, 0);
  }

  store_acc<OUT, TM, TN>(acc, Cout, ldc, M, N, m0 + wm * WM + (lane & 31), n0 + wn * WN, half,
                        OUT == kOutF32Split ? (int64_t)blockIdx.y * split_stride : 0);
}

int gemm_f32_splits(int64_t M, int64_t N, int64_t K) {
  // 128 x 128 tiles of the fp32 products: double the k-split while the units still
  // fit one round of workgroups on 256 CUs and every split keeps at least 256 k.
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int s = 1;
  while (s < 64 && tiles * s * 2 <= 256 && K / (2 * s) >= 256) s *= 2;
  return s;
}

// Explicit instantiations of every variant launched below (keeps the host-side
// launch stubs emitted for each of them).
#define SCE_GEMM_INST(T, BM, BN, AK, BK, OUT)                                              \
  template __global__ void k_gemm<T, BM, BN, AK, BK, OUT>(const T*, int64_t, const T*,     \
                                                          int64_t, void*, int64_t, int64_t, \
                                                          int64_t, int64_t, int64_t, int64_t);
SCE_GEMM_INST(float, 128, 128, true, true, kOutF32)
SCE_GEMM_INST(float, 128, 128, true, false, kOutF32)
SCE_GEMM_INST(float, 128, 128, true, false, kOutF32Split)
SCE_GEMM_INST(float, 128, 128, false, false, kOutF32Split)
#undef SCE_GEMM_INST

template <typename TIn, int BM, int BN, bool A_KC, bool B_KC, int OUT>
static hipError_t run(const GemmArgs& a, hipStream_t s) {
  constexpr int TK = Elem<TIn>::kTileK;
  const int splits = a.splits > 0 ? a.splits : 1;
  int64_t kps = (a.K + splits - 1) / splits;
  kps = (kps + TK - 1) / TK * TK;
  if (kps == 0) kps = TK;
  const int64_t gx = (a.N + BN - 1) / BN, gy = (a.M + BM - 1) / BM;
  if (gx == 0 || gy == 0) return hipGetLastError();
  if (gx * gy > 0x7fffffff || splits > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm<TIn, BM, BN, A_KC, B_KC, OUT>), dim3((unsigned)(gx * gy), splits),
                     dim3(kGemmThreads), 0, s, static_cast<const TIn*>(a.A), a.lda,
                     static_cast<const TIn*>(a.B), a.ldb, a.C, a.ldc, a.M, a.N, a.K, kps,
                     a.split_stride);
  return hipGetLastError();
}

hipError_t launch_gemm(Gemm kind, bool bf16, const GemmArgs& a, hipStream_t s) {
  if (bf16) return launch_gemm_bf16(kind, a, s);
  switch (kind) {
    case Gemm::Logits: return run<float, 128, 128, true, true, kOutF32>(a, s);
    case Gemm::DX:
      return a.splits > 1 ? run<float, 128, 128, true, false, kOutF32Split>(a, s)
                          : run<float, 128, 128, true, false, kOutF32>(a, s);
    case Gemm::DW: return run<float, 128, 128, false, false, kOutF32Split>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sce
