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

// Each lane produces 8 consecutive output elements of one dense row. With a LossOut,
// block 0 finishes the loss (alongside the copy) and the copy uses blocks 1...
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
  const int vecs_per_row = d / 8;
  const int64_t i = (int64_t)(blockIdx.x - first) * kCopyThreads + threadIdx.x;
  if (i >= (int64_t)V * vecs_per_row) return;
  const int v = (int)(i / vecs_per_row);
  const int c8 = (int)(i - (int64_t)v * vecs_per_row);
  const int p = vocab_pos ? vocab_pos[v] : v;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (p >= 0) {
    const float* src = part + (int64_t)p * d + c8 * 8;
    for (int sidx = 0; sidx < splits; ++sidx) {
      const float4 a = *reinterpret_cast<const float4*>(src + sidx * split_stride);
      const float4 b = *reinterpret_cast<const float4*>(src + sidx * split_stride + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
  }
  if (BF16) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    reinterpret_cast<uint4*>(dW)[i] = o;
  } else {
    float4* out = reinterpret_cast<float4*>(dW) + 2 * i;
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_scatter_rows(const float* part, int splits, int64_t split_stride,
                               const int32_t* vocab_pos, int V, int d, bool bf16, void* dW,
                               const LossOut* fin, hipStream_t s) {
  const int64_t total = (int64_t)V * (d / 8);
  const int blocks = (int)((total + kCopyThreads - 1) / kCopyThreads);
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
