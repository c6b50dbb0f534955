// The dense scatter of the candidate-row gradient (the row gather lives in
// kernels.h and runs inside the remap launch).
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
__device__ void finish_loss(const LossOut& f) {
  __shared__ double part[kCopyThreads / kWave];
  // Eight independent partial sums per lane keep eight loads in flight; lane l adds
  // rows l + 256 (8k + j) into partial j, and the partials are added in order j.
  constexpr int kAcc = 8;
  double a[kAcc] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int t0 = threadIdx.x; t0 < f.T; t0 += kCopyThreads * kAcc) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) {
      const int t = t0 + j * kCopyThreads;
      if (t < f.T) a[j] += (double)f.row_loss[t];
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc += a[j];
  acc = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kCopyThreads / kWave; ++w) tot += part[w];
    const int N = f.counters[kNumLabels];
    *f.loss = N > 0 ? (float)(tot / (double)N) : 0.f;
    if (f.aux) {
      f.aux[0] = f.counters[kDistinct];
      f.aux[1] = N;
      f.aux[2] = f.counters[kNextOffset];
      f.aux[3] = f.counters[kStatus];
    }
  }
}

// Each lane produces kScatterVecs vectors of 8 consecutive output elements, spaced a
// block apart so that every load of a lane is issued before its first store. With a
// LossOut, block 0 finishes the loss (alongside the copy) and the copy uses blocks 1...
// Flat vector indexes fit 32 bits: V * d / 8 <= 2^31 by the library's size limits.
constexpr int kScatterVecs = 4;
template <bool BF16>
__global__ __launch_bounds__(kCopyThreads) void k_scatter_rows(
    const float* __restrict__ part, int splits, int64_t split_stride,
    const int32_t* __restrict__ vocab_pos, int V, int d, void* __restrict__ dW, int copy_blocks,
    LossOut fin) {
  const int first = (int)gridDim.x - copy_blocks;  // 1 with a LossOut, else 0
  if ((int)blockIdx.x < first) {
    finish_loss(fin);
    return;
  }
  const uint32_t vecs_per_row = (uint32_t)d / 8;
  const uint32_t total = (uint32_t)V * vecs_per_row;
  const uint32_t i0 = (uint32_t)(blockIdx.x - first) * (kCopyThreads * kScatterVecs) + threadIdx.x;
  const float* src[kScatterVecs];
  bool live[kScatterVecs], have[kScatterVecs];
#pragma unroll
  for (int u = 0; u < kScatterVecs; ++u) {
    const uint32_t i = i0 + u * kCopyThreads;
    live[u] = i < total;
    const uint32_t v = live[u] ? i / vecs_per_row : 0;
    const uint32_t c8 = i - v * vecs_per_row;
    const int p = !live[u] ? -1 : (vocab_pos ? vocab_pos[v] : (int)v);
    have[u] = p >= 0;
    src[u] = part + (int64_t)(have[u] ? p : 0) * d + c8 * 8;
  }
  float4 lo[kScatterVecs], hi[kScatterVecs];
#pragma unroll
  for (int u = 0; u < kScatterVecs; ++u) {
    lo[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    hi[u] = lo[u];
  }
  for (int sidx = 0; sidx < splits; ++sidx) {
    float4 a[kScatterVecs], b[kScatterVecs];
#pragma unroll
    for (int u = 0; u < kScatterVecs; ++u) {
      if (have[u]) {
        a[u] = *reinterpret_cast<const float4*>(src[u] + sidx * split_stride);
        b[u] = *reinterpret_cast<const float4*>(src[u] + sidx * split_stride + 4);
      } else {
        a[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        b[u] = a[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kScatterVecs; ++u) {
      lo[u].x += a[u].x; lo[u].y += a[u].y; lo[u].z += a[u].z; lo[u].w += a[u].w;
      hi[u].x += b[u].x; hi[u].y += b[u].y; hi[u].z += b[u].z; hi[u].w += b[u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < kScatterVecs; ++u) {
    if (!live[u]) continue;
    const uint32_t i = i0 + u * kCopyThreads;
    if (BF16) {
      uint4 o;
      o.x = pack_bf16x2(lo[u].x, lo[u].y);
      o.y = pack_bf16x2(lo[u].z, lo[u].w);
      o.z = pack_bf16x2(hi[u].x, hi[u].y);
      o.w = pack_bf16x2(hi[u].z, hi[u].w);
      reinterpret_cast<uint4*>(dW)[i] = o;
    } else {
      float4* out = reinterpret_cast<float4*>(dW) + 2 * (size_t)i;
      out[0] = lo[u];
      out[1] = hi[u];
    }
  }
}

hipError_t launch_scatter_rows(const float* part, int splits, int64_t split_stride,
                               const int32_t* vocab_pos, int V, int d, bool bf16, void* dW,
                               const LossOut* fin, hipStream_t s) {
  const int64_t total = (int64_t)V * (d / 8);
  constexpr int per_block = kCopyThreads * kScatterVecs;
  const int blocks = (int)((total + per_block - 1) / per_block);
  const LossOut f = fin ? *fin : LossOut{nullptr, 0, nullptr, nullptr, nullptr};
  const int grid = blocks + (fin ? 1 : 0);
  if (grid > 0) {
    if (bf16)
      hipLaunchKernelGGL(k_scatter_rows<true>, dim3(grid), dim3(kCopyThreads), 0, s, part, splits,
                         split_stride, vocab_pos, V, d, dW, blocks, f);
    else
      hipLaunchKernelGGL(k_scatter_rows<false>, dim3(grid), dim3(kCopyThreads), 0, s, part,
                         splits, split_stride, vocab_pos, V, d, dW, blocks, f);
  }
  return hipGetLastError();
}

}  // namespace sce
