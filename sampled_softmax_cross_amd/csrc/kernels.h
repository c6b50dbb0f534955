// Launchers shared between the kernel translation units and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sce {

constexpr int kBuildThreads = 1024;
// Largest vocabulary whose candidate bitmaps (2 x V bits) the build keeps in LDS.
constexpr int kMaxBitmapClasses = 131072;

// Candidate build (P > 0: C, and the candidate bitmap `bits` and per-word prefix
// counts `wpre`, ceil(V/32) words each) or label check (P == 0), then the label remap
// and, when P > 0: with W, the row gather W_C = W[C] (rows of row_bytes, a multiple of
// 16; with WT, bf16 rows only, the gather writes W_C and its transpose WT [d, ldt],
// zeros past P, in one pass); with dW, the rows of the dense gradient outside C set to
// zero (rows of dw_row_bytes, a multiple of 16); with vocab_pos, the class -> position
// map. With amax_n >= 0 the build's launch also takes max|x| over amax_x (bf16, amax_n
// elements, a multiple of 8; null when amax_n == 0) in *amax_parts partials
// (counters[kAmaxX + i]) for launch_quant_x.
// The e4m3 step's own encoding of bf16 weights (CacheEncode given to launch_candidates):
// the build's launch also takes max|W| over W (bf16 [V, d], the `W` argument) in
// w_parts partials (counters[kAmaxW + i]); the gather then reads the bf16 rows W[C]
// (all V rows at P == 0) and writes their e4m3 codes e4m3(float32(W / s_w)),
// s_w = float32(max|W| / 448) (1 for an all-zero or non-finite W; the latter also sets
// kDevScaleRange), the rule of launch_refresh_e4m3, to W_C (rows of wc_row_bytes).
// s_w goes to *scale_slot (and *scale_out when given).
struct CacheEncode {
  int w_parts = 0;              // set by launch_candidates
  float* scale_slot = nullptr;  // device: s_w for the later kernels
  float* scale_out = nullptr;   // device or null: the caller's copy of s_w
};
hipError_t launch_candidates(const int64_t* targets, const int64_t* prefix, int T, int V, int P,
                             int stride, int off, int32_t* counters, int32_t* C, uint32_t* bits,
                             int32_t* wpre, int32_t* vocab_pos, int32_t* target_pos,
                             int32_t* prefix_pos, const void* W, int row_bytes, void* WC,
                             int wc_row_bytes, void* dW, int dw_row_bytes, hipStream_t s,
                             const void* amax_x = nullptr, int64_t amax_n = -1,
                             int* amax_parts = nullptr, void* WT = nullptr, int64_t ldt = 0,
                             CacheEncode* enc = nullptr);
hipError_t launch_write_aux(const int32_t* counters, int64_t* aux, hipStream_t s);
// The candidate stage for a set built beforehand (P > 0, V <= kMaxBitmapClasses): C_in
// [P] ascending classes and the label positions tpos_in / ppos_in (ppos_in may be null)
// are checked and copied to C / target_pos / prefix_pos, the counters set (distinct count,
// next offset and device bits from build_aux when given), then the same gather, transpose
// and zero rows as launch_candidates. amax_n >= 0: the e4m3 step's max|x| partials over
// amax_x (amax_n bf16 values) by extra workgroups of the first launch, as there.
hipError_t launch_candidates_prebuilt(const int32_t* C_in, const int32_t* tpos_in,
                                      const int32_t* ppos_in, const int64_t* build_aux, int T,
                                      int V, int P, int32_t* counters, int32_t* C, uint32_t* bits,
                                      int32_t* target_pos, int32_t* prefix_pos, const void* W,
                                      int row_bytes, void* WC, int wc_row_bytes, void* dW,
                                      int dw_row_bytes, void* WT, int64_t ldt, hipStream_t s,
                                      const void* amax_x = nullptr, int64_t amax_n = -1,
                                      int* amax_parts = nullptr);

// Row gather, one block of 256 lanes per kGatherRows rows: 32 lanes per row, each
// moving whole 16-byte vectors, every load of a lane issued before its stores. Rows of
// W are row_vecs vectors apart, rows of W_C wc_vecs (>= row_vecs) apart.
constexpr int kGatherRows = 8;
inline int gather_block_count(int P, int row_vecs) {
  (void)row_vecs;
  return (P + kGatherRows - 1) / kGatherRows;
}
__device__ __forceinline__ void gather_rows_block(int blk, const uint4* __restrict__ W,
                                                  const int32_t* __restrict__ C, int P,
                                                  int row_vecs, uint4* __restrict__ WC,
                                                  int wc_vecs) {
  const int r = blk * kGatherRows + (int)(threadIdx.x >> 5);
  if (r >= P) return;
  const int l = threadIdx.x & 31;
  const uint4* src = W + (int64_t)C[r] * row_vecs;
  uint4* dst = WC + (int64_t)r * wc_vecs;
  for (int v0 = l; v0 < row_vecs; v0 += 32 * 4) {
    const bool k1 = v0 + 32 < row_vecs, k2 = v0 + 64 < row_vecs, k3 = v0 + 96 < row_vecs;
    uint4 b1 = make_uint4(0, 0, 0, 0), b2 = b1, b3 = b1;
    const uint4 b0 = src[v0];
    if (k1) b1 = src[v0 + 32];
    if (k2) b2 = src[v0 + 64];
    if (k3) b3 = src[v0 + 96];
    dst[v0] = b0;
    if (k1) dst[v0 + 32] = b1;
    if (k2) dst[v0 + 64] = b2;
    if (k3) dst[v0 + 96] = b3;
  }
}
// e4m3 codes of 8 bf16 values over s_w: W / s_w correctly rounded (float division),
// clamped to [-448, 448] (every value in [448, 464) encodes as 448, and s_w rounded below
// max|W| / 448 can put the largest quotient a rounding error above 448), round to
// nearest even.
__device__ __forceinline__ uint2 encode_e4m3x8(const uint4& q, float s_w) {
  auto quo = [s_w](float w) { return fminf(fmaxf(w / s_w, -448.f), 448.f); };
  uint2 o;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(quo(__uint_as_float(q.x << 16)),
                                          quo(__uint_as_float(q.x & 0xffff0000u)), 0, false);
  o.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quo(__uint_as_float(q.y << 16)),
                                                  quo(__uint_as_float(q.y & 0xffff0000u)), w, true);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(quo(__uint_as_float(q.z << 16)),
                                      quo(__uint_as_float(q.z & 0xffff0000u)), 0, false);
  o.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quo(__uint_as_float(q.w << 16)),
                                                  quo(__uint_as_float(q.w & 0xffff0000u)), w, true);
  return o;
}
// The gather with encoding: rows r of block blk (kGatherRows of them, 32 lanes each) read
// bf16 row map ? map[r] : r of W (row_vecs 16-byte vectors) and write its e4m3 codes to
// row r of WC (wc_bytes apart), every load of a lane issued before its stores.
__device__ __forceinline__ void gather_encode_block(int blk, const uint4* __restrict__ W,
                                                    const int32_t* __restrict__ map, int rows,
                                                    int row_vecs, uint8_t* __restrict__ WC,
                                                    int64_t wc_bytes, float s_w) {
  const int r = blk * kGatherRows + (int)(threadIdx.x >> 5);
  if (r >= rows) return;
  const int l = threadIdx.x & 31;
  const uint4* src = W + (int64_t)(map ? map[r] : r) * row_vecs;
  uint2* dst = reinterpret_cast<uint2*>(WC + (int64_t)r * wc_bytes);
  for (int v0 = l; v0 < row_vecs; v0 += 32 * 4) {
    uint4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = v0 + 32 * j;
      q[j] = src[v < row_vecs ? v : v0];  // past the row: a vector it has (not stored)
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v0 + 32 * j < row_vecs) dst[v0 + 32 * j] = encode_e4m3x8(q[j], s_w);
  }
}

// Tiled transpose through LDS: one block of 256 lanes moves the kTrTile x kTrTile tile
// (bx, by) of dst[c, r] = src[map ? map[r] : r, c] (r < rows, c < cols; dst columns r in
// [rows, ld_dst) get zeros). It reads 16-byte chunks along the source rows and writes
// 16-byte chunks along the destination rows, so both sides stay coalesced; the LDS rows
// are padded by one 4-byte word so the column-wise reads of a chunk fall on different
// banks. With `copy`, the rows it read also go to copy[r, c] (the gathered rows, for a
// gather that also transposes: its source is read once for both).
constexpr int kTrTile = 64;
template <typename E>
__device__ __forceinline__ void transpose_tile(int bx, int by, const E* __restrict__ src,
                                               int64_t ld_src, const int32_t* __restrict__ map,
                                               int rows, int cols, E* __restrict__ dst,
                                               int64_t ld_dst, E* __restrict__ copy,
                                               int64_t ld_copy) {
  constexpr int EPC = 16 / sizeof(E);           // elements per 16-byte chunk
  constexpr int CPR = kTrTile / EPC;            // chunks per tile row
  constexpr int LDT = kTrTile + 4 / sizeof(E);  // padded LDS row (elements)
  __shared__ E tile[kTrTile * LDT];
  const int r0 = bx * kTrTile, c0 = by * kTrTile;
  for (int q = threadIdx.x; q < kTrTile * CPR; q += 256) {
    const int r = q / CPR, c = (q % CPR) * EPC;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < rows && c0 + c < cols) {
      const int64_t sr = map ? (int64_t)map[r0 + r] : (int64_t)(r0 + r);
      v = *reinterpret_cast<const uint4*>(src + sr * ld_src + c0 + c);
      if (copy) *reinterpret_cast<uint4*>(copy + (int64_t)(r0 + r) * ld_copy + c0 + c) = v;
    }
    const E* e = reinterpret_cast<const E*>(&v);
#pragma unroll
    for (int i = 0; i < EPC; ++i) tile[r * LDT + c + i] = e[i];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTrTile * CPR; q += 256) {
    const int c = q / CPR, r = (q % CPR) * EPC;  // destination row c, columns r .. r + EPC
    if (c0 + c >= cols || r0 + r >= ld_dst) continue;
    uint4 v;
    E* e = reinterpret_cast<E*>(&v);
#pragma unroll
    for (int i = 0; i < EPC; ++i) e[i] = tile[(r + i) * LDT + c];
    *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + c) * ld_dst + r0 + r) = v;
  }
}

// Zero rows of the dense gradient: block `blk` covers kZeroVecs 16-byte vectors of the
// flat [V, vpr] array (vpr vectors per row) and clears those of rows outside C (bit
// clear in the candidate bitmap): one lookup per vector, all four of a lane issued
// before the first is tested (a vector past the end looks up row 0), then stores only.
constexpr int kZeroVecs = 256 * 4;
inline int zero_block_count(int V, int vpr) {
  return (int)(((int64_t)V * vpr + kZeroVecs - 1) / kZeroVecs);
}
__device__ __forceinline__ void zero_rows_block(int blk, const uint32_t* __restrict__ bits, int V,
                                                int vpr, uint4* __restrict__ dW) {
  const int64_t total = (int64_t)V * vpr;
  const int64_t i0 = (int64_t)blk * kZeroVecs + threadIdx.x;
  uint32_t word[4];
  int row[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + u * 256;
    row[u] = i < total ? (int)(i / vpr) : 0;
    word[u] = bits[row[u] >> 5];
  }
  bool in_c[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) in_c[u] = i0 + u * 256 >= total || ((word[u] >> (row[u] & 31)) & 1u);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (!in_c[u]) dW[i0 + u * 256] = make_uint4(0, 0, 0, 0);
}
// dW[C[p], :] = sum over splits of part[s, p, :] (fp32) in dtype for p < rows (C null:
// the identity). When `fin` is given, the launch also finishes the step's scalars:
// loss = sum(row_loss[0..T)) / N in a fixed order (0 when N == 0) and, when aux is
// given, the counters.
struct LossOut {
  const float* row_loss;
  int T;
  const int32_t* counters;
  float* loss;
  int64_t* aux;
};
hipError_t launch_scatter_rows(const float* part, int splits, int64_t split_stride,
                               const int32_t* C, int rows, int d, bool bf16, void* dW,
                               const LossOut* fin, hipStream_t s);

// Caller-given label positions for the CE alone: copies with positions outside
// [-1, P) replaced by -1 (flagged in the status counter), N counted, counters set.
hipError_t launch_ce_prep(const int32_t* tpos_in, const int32_t* ppos_in, int T, int P,
                          int32_t* tpos, int32_t* ppos, int32_t* counters, hipStream_t s);
// out[i, :] = W[idx[i], :] (zeros and kDevLabelRange in *status for idx outside [0, V)).
// dst[c, r] = src[r, c] for r < rows, c < cols, elements of es bytes (1 or 2); dst
// columns r in [rows, ld_dst) are written as zeros. src rows are ld_src elements apart,
// dst rows ld_dst; both pitches and cols keep every 16-byte chunk whole (multiples of
// 16 / es).
hipError_t launch_transpose(const void* src, int64_t ld_src, int rows, int cols, int es, void* dst,
                            int64_t ld_dst, hipStream_t s);
hipError_t launch_gather_checked(const void* W, int64_t V, const int32_t* idx, int n,
                                 int row_bytes, void* out, int64_t out_row_bytes,
                                 int32_t* status, hipStream_t s);

// Row-wise cross-entropy forward/backward over Z [T, ldz] (P valid columns), in place.
hipError_t launch_ce_rows(void* Z, int64_t ldz, int T, int P, bool bf16,
                          const int32_t* target_pos, const int32_t* prefix_pos,
                          const int32_t* counters, float* row_loss, float* row_lse,
                          hipStream_t s);
// e4m3 step: the same over bf16 Z, with the gradient written as e4m3 codes of g / s_g
// to its own buffer (Z is left as it is) and s_g derived from N.
struct G8Out {
  uint8_t* g8;        // [T, ldg] codes; every column below ldz is written, those in
                      // [P, ldz) as zero codes: the e4m3 products read 16-element chunks
                      // that straddle K = P and rely on those zeros
  int64_t ldg;        // equal to ldz (a multiple of 16; checked by the launcher)
  int n_max;          // labels per row at most: 1, or 2 with prefix targets
  float* scales;      // the step's scale table (reads kScaleX, kScaleW; writes the rest)
  float* scales_out;  // caller's {s_x, s_g}, or null (writes [1])
};
hipError_t launch_ce_rows_g8(const void* Z, int64_t ldz, int T, int P, const int32_t* target_pos,
                             const int32_t* prefix_pos, const int32_t* counters, float* row_loss,
                             float* row_lse, const G8Out& go, hipStream_t s);

// e4m3 step: s_x from max|x| over bf16 x [n] (n a multiple of 8), and x8 = e4m3(x / s_x)
// (bytes, same layout); fills the scale table's x entries (the cache's scale: *w_scale_dev
// when given, else w_scale; and s_x) and scales_out[0] when given. max|x| comes from the amax_parts partials that
// launch_candidates left in counters[kAmaxX ...] (amax_parts > 0), else from an amax
// launch of its own.
hipError_t launch_quant_x(const void* x, int64_t n, int32_t* counters, float w_scale,
                          const float* w_scale_dev, void* x8, float* scales, float* scales_out,
                          hipStream_t s, int amax_parts = 0);
// The e4m3 lm_head cache refresh: W8 = e4m3(W / s_w), s_w = max|W| / 448 (float32; 1 for an
// all-zero W) written to *scale_out, over n bf16 values (a multiple of 8). part: kAmaxX +
// kAmaxSlots ints of scratch for the per-workgroup maxima; status (may be null) is set to 0, or to
// kDevScaleRange when W holds a non-finite value.
hipError_t launch_refresh_e4m3(const void* W, int64_t n, void* W8, float* scale_out,
                               int32_t* status, int32_t* part, hipStream_t s);

// max|x| partial of one amax block (kBuildThreads lanes; block `b` of `nb`) over nvec
// 16-byte bf16 vectors, written as the magnitude's bits to counters[kAmaxX + b]. LOADS
// vectors per lane and round. Beside the candidate build, 16 (kAmaxLoadsBuild): max|x|
// and max|W| of the stage-0/1 e4m3 step (102 MB) take 392 blocks, one round beside the
// build (8 loads: 782 blocks, 1.5 rounds, and a candidate stage 2.3 us longer). Alone
// (the cache refresh), 8 (kAmaxLoads): max|W| in 589 blocks, 15.7 us on average against
// 18.1 us in 295 blocks, which spread unevenly over 256 CUs.
constexpr int kAmaxLoads = 8, kAmaxLoadsBuild = 16;
template <int LOADS = kAmaxLoads>
inline int amax_block_count(int64_t nvec) {
  const int64_t want = (nvec + (int64_t)kBuildThreads * LOADS - 1) / ((int64_t)kBuildThreads * LOADS);
  return (int)(want < 1 ? 1 : (want > kAmaxSlots ? kAmaxSlots : want));
}
// Magnitude bits of the largest |x| of 8 bf16 values (bf16 magnitudes order like their
// bit patterns).
__device__ __forceinline__ uint32_t amax8(const uint4& q) {
  uint32_t m = 0;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7fffu);
    m = max(m, (w[i] >> 16) & 0x7fffu);
  }
  return m;
}
// Each block writes the largest magnitude it saw to its own partial (no atomics:
// atomics on one address serialise, one per workgroup of 512 measured 10.8 us for a
// 25 MB tensor); LOADS loads in flight per lane, all issued before the first use.
template <int LOADS = kAmaxLoads>
__device__ __forceinline__ void amax_bf16_block(const uint4* __restrict__ x, int64_t nvec, int b,
                                                int nb, int32_t* __restrict__ counters) {
  __shared__ uint32_t wmax[kBuildThreads / 64];
  uint32_t m = 0;
  const int64_t stride = (int64_t)nb * kBuildThreads;
  for (int64_t i0 = (int64_t)b * kBuildThreads + threadIdx.x; i0 < nvec; i0 += LOADS * stride) {
    uint4 q[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int64_t i = i0 + j * stride;
      q[j] = x[i < nvec ? i : nvec - 1];  // past the end: the last vector again (no change)
    }
#pragma unroll
    for (int j = 0; j < LOADS; ++j) m = max(m, amax8(q[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kBuildThreads / 64; ++w) t = max(t, wmax[w]);
    counters[kAmaxX + b] = (int32_t)t;
  }
}


// GEMMs. Matrices row-major; see gemm.hip for the operand conventions.
enum class Gemm { Logits, DX, DW };
// The dW product's two kinds of unit (kOutDW). The tile order is row-major over
// nbx <= 4 column tiles; its first `whole` tiles (a multiple of nbx: whole row blocks,
// rows [0, r0)) are computed over all of K by one unit each and stored as bf16 straight
// into the dense gradient, at row rowmap[row] (the candidate class; row itself when
// rowmap is null). The other tiles are k-split as usual into fp32 partial slabs of rows
// [r0, M) (partial row = row - r0), which a reduction sums and scatters. Whole units fill
// the chip in whole rounds and only the tiles left over are split, so the partial round
// trip covers those alone.
struct DwOut {
  void* dW = nullptr;             // bf16 rows of ldw elements
  int64_t ldw = 0;
  const int32_t* rowmap = nullptr;
  int whole = 0;
  int64_t r0 = 0;
};
struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int64_t M, N, K;
  int splits;            // split-K factor (fp32 partial slabs when > 1)
  int64_t split_stride;  // elements between split slabs of C
  const float* scale = nullptr;  // e4m3 products: device factor applied before the store
  DwOut dw{};                    // dW with whole tiles (dw.whole > 0): see DwOut
};
// The schedule of the bf16 / e4m3 dW product (M = P, N = d, K = T): `whole` tiles
// computed whole and stored into dW (rows [0, r0) of the candidate order), the rest
// k-split `splits` ways into fp32 partials of rows [r0, M). whole = 0, r0 = 0: every
// tile split (splits = 1: one fp32 slab).
struct DwPlan {
  int splits = 1;
  int whole = 0;
  int64_t r0 = 0;
};
DwPlan gemm_bf16_dw_plan(int64_t M, int64_t N, int64_t K);
DwPlan gemm_fp8_dw_plan(int64_t M, int64_t N, int64_t K);
int gemm_fp8_dx_splits(int64_t M, int64_t N, int64_t K);
int gemm_bf16_dx_splits(int64_t M, int64_t N, int64_t K);
int gemm_f32_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(Gemm kind, bool bf16, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16(Gemm kind, const GemmArgs& a, hipStream_t s);
// e4m3 operands (A, B as bytes; a.scale required), fp32 accumulation.
hipError_t launch_gemm_fp8(Gemm kind, const GemmArgs& a, hipStream_t s);

}  // namespace sce
