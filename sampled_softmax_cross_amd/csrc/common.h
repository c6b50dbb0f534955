// Shared device helpers for the sampled-CE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sce {

constexpr int kWave = 64;

// Workspace counters (int32), cleared by the first kernel of every call.
enum Counter : int {
  kStatus = 0,     // SCE_DEV_* bits
  kNumLabels = 1,  // N: labels whose position is >= 0
  kDistinct = 2,   // distinct targets
  kNextOffset = 3, // sweep offset after the build
  kCeDone = 4,     // CE rows finished (the last one reduces the loss)
  kNumCounters = 8,
  // After the counters (not cleared with them): the e4m3 step's bf16 magnitude bits of
  // max|x|, one partial per workgroup of the amax launch (at most kAmaxSlots), then
  // those of max|W| when the step encodes the candidate rows of bf16 weights itself.
  kAmaxX = kNumCounters,
  kAmaxSlots = 1024,
  kAmaxW = kAmaxX + kAmaxSlots,
  kCounterWords = kAmaxW + kAmaxSlots
};
constexpr int kDevTooManyTargets = 1;
constexpr int kDevLabelRange = 2;
constexpr int kDevScaleRange = 4;

// e4m3 step: the scale table in the workspace (floats). The three products' output
// factors, and the per-tensor scales they are made of.
enum Scale : int {
  kScaleLogits = 0,  // s_x * w_scale
  kScaleDx = 1,      // s_g * w_scale
  kScaleDw = 2,      // s_g * s_x
  kScaleX = 3,       // s_x
  kScaleG = 4,       // s_g
  kScaleW = 5,       // w_scale
  kScaleWCache = 6,  // s_w formed by the step from bf16 weights (read as a device w_scale)
  kNumScales = 8
};

// bfloat16 is carried as its 16 raw bits.
using bf16_t = uint16_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bfloat16 for two values packed into one dword
// (lo in bits 0..15). gfx950 has a native instruction for this.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// ---- wave / block reductions (wave64) ----
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum across a wave (Hillis-Steele over lane ids).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive prefix sum across the block; returns the block total in *total.
// `scratch` holds at least blockDim.x / 64 + 1 ints of shared memory. Contains
// barriers: every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    int t = lane < nw ? scratch[lane] : 0;
    int ti = wave_inclusive_scan(t);
    if (lane < nw) scratch[lane] = ti - t;  // exclusive wave offsets
    if (lane == nw - 1) scratch[nw] = ti;   // block total
  }
  __syncthreads();
  int r = scratch[wid] + inc - v;
  *total = scratch[nw];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_sum_int(int v, int* scratch) {
  int total;
  (void)block_exclusive_scan(v, scratch, &total);
  return total;
}

}  // namespace sce
