// The dense scatter of the candidate-row gradient, and the row gather on its own (the
// step's gather lives in kernels.h and runs inside the remap launch).
//
// Both are pure data movement ("sampled_softmax.py", SampledSoftmax._gather_rows
// copies the candidates' lm_head rows into a contiguous [P, d] table; the module
// docstring makes the lm_head gradient dense with zeros outside C). They are
// written as flat, 16-byte-vectorised, fully coalesced copies: every lane moves
// whole 16-byte vectors and consecutive lanes touch consecutive addresses, which
// is all a bandwidth-bound copy needs (the index-select review on torchtitan
// PR #1083 reaches the same conclusion: plain vectorised loads and stores with 1-D
// blocking, nothing to hide with asynchronous copies).
#include "common.h"
#include "kernels.h"

namespace sce {

constexpr int kCopyThreads = 256;

// loss = sum of the rows' loss terms / N, summed by one block in a fixed order.
// Each lane issues all the loads of a round (kLossRows rows, a block apart: 8192
// rows per round) before its first add, which it makes in row order. The loads are
// unconditional (rows past T read row T - 1 and count as zero): a load under a
// branch would have its conversion placed in the same branch, behind a wait for that
// one load, which turns the round into kLossRows round trips to memory.
constexpr int kLossRows = 32;
__device__ void finish_loss(const LossOut& f) {
  __shared__ double part[kCopyThreads / kWave];
  // the counters travel with the first round of loads
  const int N = f.counters[kNumLabels], distinct = f.counters[kDistinct],
            next_off = f.counters[kNextOffset], status = f.counters[kStatus];
  double acc = 0.0;
  for (int t0 = threadIdx.x; t0 < f.T; t0 += kCopyThreads * kLossRows) {
    float v[kLossRows];
#pragma unroll
    for (int j = 0; j < kLossRows; ++j) {
      const int t = t0 + j * kCopyThreads;
      const float x = f.row_loss[t < f.T ? t : f.T - 1];
      v[j] = t < f.T ? x : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kLossRows; ++j) acc += (double)v[j];
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kCopyThreads / kWave; ++w) tot += part[w];
    *f.loss = N > 0 ? (float)(tot / (double)N) : 0.f;
    if (f.aux) {
      f.aux[0] = distinct;
      f.aux[1] = N;
      f.aux[2] = next_off;
      f.aux[3] = status;
    }
  }
}

// One launch, two roles by block index:
//  * with a LossOut, block 0 finishes the loss;
//  * row blocks write the candidate rows: dW[C[p], :] = sum over splits of
//    part[s, p, :], with C = identity when no map is given. Their loads depend on
//    nothing, the candidate's class only addresses the store.
// (The rows outside C are cleared earlier, by the label-remap launch.)
// Each lane handles kScatterVecs vectors of 8 consecutive elements, a block apart,
// every load issued before the first store. Flat vector indexes fit 32 bits: V * d / 8
// and T * d / 8 are at most 2^31 by the library's size limits.
constexpr int kScatterVecs = 4;
constexpr int kPerBlock = kCopyThreads * kScatterVecs;

template <bool BF16>
__device__ __forceinline__ void store_vec(void* dW, size_t i, const float4& lo, const float4& hi) {
  if (BF16) {
    uint4 o;
    o.x = pack_bf16x2(lo.x, lo.y);
    o.y = pack_bf16x2(lo.z, lo.w);
    o.z = pack_bf16x2(hi.x, hi.y);
    o.w = pack_bf16x2(hi.z, hi.w);
    reinterpret_cast<uint4*>(dW)[i] = o;
  } else {
    float4* out = reinterpret_cast<float4*>(dW) + 2 * i;
    out[0] = lo;
    out[1] = hi;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kCopyThreads) void k_scatter_rows(
    const float* __restrict__ part, int splits, int64_t split_stride, const int32_t* __restrict__ C,
    int rows, int d, void* __restrict__ dW, int row_blocks, LossOut fin) {
  const int first = (int)gridDim.x - row_blocks;  // 1 with a LossOut, else 0
  const int b = (int)blockIdx.x - first;
  if (b < 0) {
    finish_loss(fin);
    return;
  }
  const uint32_t vpr = (uint32_t)d / 8;
  const uint32_t total = (uint32_t)rows * vpr;
  const uint32_t i0 = (uint32_t)b * kPerBlock + threadIdx.x;
  // Destination rows first, loaded unconditionally (a vector past the end takes the
  // last one's row and is not stored), so the class loads travel with the others
  // rather than each waiting alone in front of its store.
  uint32_t dst[kScatterVecs];
#pragma unroll
  for (int u = 0; u < kScatterVecs; ++u) {
    const uint32_t i = i0 + u * kCopyThreads;
    const uint32_t ic = i < total ? i : total - 1;
    const uint32_t p = ic / vpr, c8 = ic - p * vpr;
    dst[u] = (C ? (uint32_t)C[p] : p) * vpr + c8;
  }
  float4 lo[kScatterVecs], hi[kScatterVecs];
#pragma unroll
  for (int u = 0; u < kScatterVecs; ++u) {
    lo[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    hi[u] = lo[u];
  }
  for (int sidx = 0; sidx < splits; ++sidx) {
    float4 a[kScatterVecs], c[kScatterVecs];
#pragma unroll
    for (int u = 0; u < kScatterVecs; ++u) {
      const uint32_t i = i0 + u * kCopyThreads;
      const float* src = part + sidx * split_stride + (size_t)i * 8;
      if (i < total) {
        a[u] = *reinterpret_cast<const float4*>(src);
        c[u] = *reinterpret_cast<const float4*>(src + 4);
      } else {
        a[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        c[u] = a[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kScatterVecs; ++u) {
      lo[u].x += a[u].x; lo[u].y += a[u].y; lo[u].z += a[u].z; lo[u].w += a[u].w;
      hi[u].x += c[u].x; hi[u].y += c[u].y; hi[u].z += c[u].z; hi[u].w += c[u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < kScatterVecs; ++u)
    if (i0 + u * kCopyThreads < total) store_vec<BF16>(dW, dst[u], lo[u], hi[u]);
}

// out[i, :] = W[idx[i], :] for i < n (rows of row_vecs 16-byte vectors, out rows
// out_vecs apart); an index outside [0, V) gives a row of zeros and sets
// kDevLabelRange in *status when status is given. 32 lanes per row, as the gather of
// the step.
__global__ __launch_bounds__(256) void k_gather_checked(const uint4* __restrict__ W, int64_t V,
                                                        const int32_t* __restrict__ idx, int n,
                                                        int row_vecs, uint4* __restrict__ out,
                                                        int64_t out_vecs,
                                                        int32_t* __restrict__ status) {
  const int r = (int)blockIdx.x * kGatherRows + (int)(threadIdx.x >> 5);
  if (r >= n) return;
  const int l = threadIdx.x & 31;
  const int64_t c = idx[r];
  uint4* dst = out + (int64_t)r * out_vecs;
  if (c < 0 || c >= V) {
    for (int v = l; v < row_vecs; v += 32) dst[v] = make_uint4(0, 0, 0, 0);
    if (status && l == 0) atomicOr(status, kDevLabelRange);
    return;
  }
  const uint4* src = W + c * row_vecs;
  // kInFlight vectors per lane per round, every load before the first store.
  constexpr int kInFlight = 8;
  for (int v0 = l; v0 < row_vecs; v0 += 32 * kInFlight) {
    uint4 b[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      b[u] = v0 + 32 * u < row_vecs ? src[v0 + 32 * u] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      if (v0 + 32 * u < row_vecs) dst[v0 + 32 * u] = b[u];
  }
}

hipError_t launch_gather_checked(const void* W, int64_t V, const int32_t* idx, int n,
                                 int row_bytes, void* out, int64_t out_row_bytes,
                                 int32_t* status, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_gather_checked, dim3((n + kGatherRows - 1) / kGatherRows), dim3(256), 0,
                       s, static_cast<const uint4*>(W), V, idx, n, row_bytes / 16,
                       static_cast<uint4*>(out), out_row_bytes / 16, status);
  return hipGetLastError();
}

// Tiled transpose through LDS (transpose_tile in kernels.h), one tile per block.
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E* __restrict__ src, int64_t ld_src,
                                                   int rows, int cols, E* __restrict__ dst,
                                                   int64_t ld_dst) {
  transpose_tile<E>((int)blockIdx.x, (int)blockIdx.y, src, ld_src, nullptr, rows, cols, dst, ld_dst,
                    nullptr, 0);
}

hipError_t launch_transpose(const void* src, int64_t ld_src, int rows, int cols, int es, void* dst,
                            int64_t ld_dst, hipStream_t s) {
  const dim3 grid((unsigned)((ld_dst + kTrTile - 1) / kTrTile), (unsigned)((cols + kTrTile - 1) / kTrTile));
  if (grid.x == 0 || grid.y == 0) return hipGetLastError();
  if (es == 2)
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src),
                       ld_src, rows, cols, static_cast<uint16_t*>(dst), ld_dst);
  else
    hipLaunchKernelGGL(k_transpose<uint8_t>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(src),
                       ld_src, rows, cols, static_cast<uint8_t*>(dst), ld_dst);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* part, int splits, int64_t split_stride,
                               const int32_t* C, int rows, int d, bool bf16, void* dW,
                               const LossOut* fin, hipStream_t s) {
  const int64_t vpr = d / 8;
  const int row_blocks = (int)(((int64_t)rows * vpr + kPerBlock - 1) / kPerBlock);
  const LossOut f = fin ? *fin : LossOut{nullptr, 0, nullptr, nullptr, nullptr};
  const int grid = row_blocks + (fin ? 1 : 0);
  if (grid > 0) {
    if (bf16)
      hipLaunchKernelGGL(k_scatter_rows<true>, dim3(grid), dim3(kCopyThreads), 0, s, part, splits,
                         split_stride, C, rows, d, dW, row_blocks, f);
    else
      hipLaunchKernelGGL(k_scatter_rows<false>, dim3(grid), dim3(kCopyThreads), 0, s, part,
                         splits, split_stride, C, rows, d, dW, row_blocks, f);
  }
  return hipGetLastError();
}

}  // namespace sce
