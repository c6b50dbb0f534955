// Row gather W_C = W[C] and the dense scatter of the candidate-row gradient.
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
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void k_gather_rows(const uint4* __restrict__ W,
                                                              const int32_t* __restrict__ C,
                                                              int P, int row_vecs,
                                                              uint4* __restrict__ WC) {
  const int total = P * row_vecs;
  const int base = blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  uint4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int i = base + u * kCopyThreads;
    if (i < total) {
      const int r = i / row_vecs;
      const int k = i - r * row_vecs;
      v[u] = W[(int64_t)C[r] * row_vecs + k];
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int i = base + u * kCopyThreads;
    if (i < total) WC[i] = v[u];
  }
}

hipError_t launch_gather_rows(const void* W, const int32_t* C, int P, int row_bytes, void* WC,
                              hipStream_t s) {
  const int row_vecs = row_bytes / 16;
  const int64_t total = (int64_t)P * row_vecs;
  const int blocks = (int)((total + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll));
  if (blocks > 0)
    hipLaunchKernelGGL(k_gather_rows, dim3(blocks), dim3(kCopyThreads), 0, s,
                       reinterpret_cast<const uint4*>(W), C, P, row_vecs,
                       reinterpret_cast<uint4*>(WC));
  return hipGetLastError();
}

// Each lane produces 8 consecutive output elements of one dense row.
template <bool BF16>
__global__ __launch_bounds__(kCopyThreads) void k_scatter_rows(
    const float* __restrict__ part, int splits, int64_t split_stride,
    const int32_t* __restrict__ vocab_pos, int V, int d, void* __restrict__ dW) {
  const int vecs_per_row = d / 8;
  const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
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
                               hipStream_t s) {
  const int64_t total = (int64_t)V * (d / 8);
  const int blocks = (int)((total + kCopyThreads - 1) / kCopyThreads);
  if (blocks > 0) {
    if (bf16)
      hipLaunchKernelGGL(k_scatter_rows<true>, dim3(blocks), dim3(kCopyThreads), 0, s, part,
                         splits, split_stride, vocab_pos, V, d, dW);
    else
      hipLaunchKernelGGL(k_scatter_rows<false>, dim3(blocks), dim3(kCopyThreads), 0, s, part,
                         splits, split_stride, vocab_pos, V, d, dW);
  }
  return hipGetLastError();
}

}  // namespace sce
