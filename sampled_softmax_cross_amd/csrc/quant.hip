// Per-tensor e4m3 quantisation of the activations x (bf16 [T, d]) for the fp8 step.
//
// The lm_head rows of "sampled_softmax.py" are an e4m3 cache and the products are
// scaled fp8 products; x is quantised here with a power-of-two scale: s_x is the
// smallest power of two with max|x| <= 448 s_x (448: the largest finite e4m3 value),
// so x / s_x is exact and the conversion (round to nearest even, OCP E4M3, the
// hardware's v_cvt_pk_fp8_f32) is the only rounding.
//
// The amax of |x| over the whole tensor (per-workgroup maxima of the bf16 magnitude
// bits, which order like the values) is taken by extra workgroups of the candidate
// build's launch (amax_bf16_block), which runs on one workgroup and leaves the rest of
// the chip idle; the conversion's workgroups each reduce those maxima, derive s_x from
// the amax in integers and write the step's scale table.
#include "common.h"
#include "kernels.h"

namespace sce {

// s_x = 2^e from the bf16 magnitude bits of max|x|: with max|x| = f 2^E, f in [0.5, 1),
// 448 2^e = 0.875 2^(e + 9) covers it first at e = E - 9 when f <= 0.875, else at
// e = E - 8. f <= 0.875 is a mantissa (7 bits) of at most 0x60 (1.75 = 1 + 96/128).
// Returns false for magnitudes outside the path's range (non-finite, or nonzero below
// 2^-100, where 1 / s_x would leave float range).
__device__ __forceinline__ bool x_scale_exponent(uint32_t abits, int& e) {
  if (abits == 0) {
    e = 0;
    return true;
  }
  const int ef = (int)(abits >> 7);  // biased exponent
  if (ef >= 255 || ef < 127 - 100) return false;
  const int E = ef - 126;
  e = (abits & 0x7f) <= 0x60 ? E - 9 : E - 8;
  return true;
}

__device__ __forceinline__ float pow2f(int e) { return __int_as_float((127 + e) << 23); }

__global__ __launch_bounds__(256) void k_quant_e4m3(const uint4* __restrict__ x, int64_t nvec,
                                                    int32_t* __restrict__ counters, int npart,
                                                    float w_scale_host,
                                                    const float* __restrict__ w_scale_dev,
                                                    uint2* __restrict__ x8,
                                                    float* __restrict__ scales,
                                                    float* __restrict__ scales_out) {
  // the cache's scale: a device value (read in stream order, e.g. after a refresh), or
  // the caller's host value; a device value that is not positive and finite is flagged
  const float w_scale = w_scale_dev ? *w_scale_dev : w_scale_host;
  const bool w_ok = w_scale > 0.f && w_scale <= 3.0e38f;
  // max|x| from the amax launch's npart partials (L2-resident, 4 per lane at most)
  __shared__ uint32_t wmax[256 / kWave];
  uint32_t amax = 0;
  for (int i = threadIdx.x; i < npart; i += 256) amax = max(amax, (uint32_t)counters[kAmaxX + i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  int e = 0;
  const bool ok = x_scale_exponent(amax, e);
  if (!ok) e = 0;
  const float inv = pow2f(-e);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const float sx = pow2f(e);
    scales[kScaleLogits] = sx * w_scale;
    scales[kScaleX] = sx;
    scales[kScaleW] = w_scale;
    // s_g = 1 until the cross-entropy (which derives it from N) runs: T = 0 keeps these
    scales[kScaleG] = 1.f;
    scales[kScaleDx] = w_scale;
    scales[kScaleDw] = sx;
    if (scales_out) {
      scales_out[0] = sx;
      scales_out[1] = 1.f;
    }
    if (!ok || !w_ok) atomicOr(&counters[kStatus], kDevScaleRange);
  }
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
    const uint4 q = x[i];
    uint2 o;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(q.x) * inv, bf16_hi(q.x) * inv, 0, false);
    o.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(q.y) * inv, bf16_hi(q.y) * inv, w, true);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(q.z) * inv, bf16_hi(q.z) * inv, 0, false);
    o.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(q.w) * inv, bf16_hi(q.w) * inv, w, true);
    x8[i] = o;
  }
}

hipError_t launch_quant_x(const void* x, int64_t n, int32_t* counters, float w_scale,
                          const float* w_scale_dev, void* x8, float* scales, float* scales_out,
                          hipStream_t s, int amax_parts) {
  if (amax_parts < 1 || amax_parts > kAmaxSlots) return hipErrorInvalidValue;
  const int64_t nvec = n / 8;
  const int64_t want = (nvec + 255) / 256;
  const int grid = (int)(want < 2048 ? (want > 0 ? want : 1) : 2048);
  hipLaunchKernelGGL(k_quant_e4m3, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(x), nvec,
                     counters, amax_parts, w_scale, w_scale_dev, static_cast<uint2*>(x8), scales,
                     scales_out);
  return hipGetLastError();
}

// ---- the e4m3 lm_head cache refresh --------------------------------------------------
// W (bf16 [V, d]) -> codes e4m3(W / s_w) with s_w = max|W| / 448 in float32 (1 when W is
// all zeros): the largest magnitude maps to e4m3's largest finite value. The quotient is
// the correctly rounded float32 division and the encoding rounds to nearest even, so the
// codes are exactly those of float32(W / s_w) cast to OCP E4M3.

// W / s_w, correctly rounded (hipcc's float division is, unless fast-math is asked for),
// clamped to [-448, 448]: s_w = float32(max|W| / 448) can fall below the exact quotient, so
// max|W| / s_w can exceed 448 by a rounding error (at most 448 (1 + 2^-23)); every value in
// [448, 464) rounds to 448 in e4m3, so the clamp changes no code and keeps the conversion
// off its out-of-range inputs.
__device__ __forceinline__ float cache_quotient(float w, float s_w) {
  return fminf(fmaxf(w / s_w, -448.f), 448.f);
}

__global__ __launch_bounds__(kBuildThreads) void k_amax_w(const uint4* __restrict__ W,
                                                          int64_t nvec,
                                                          int32_t* __restrict__ part) {
  amax_bf16_block(W, nvec, (int)blockIdx.x, (int)gridDim.x, part);
}

__global__ __launch_bounds__(256) void k_refresh_e4m3(const uint4* __restrict__ W, int64_t nvec,
                                                      const int32_t* __restrict__ part, int npart,
                                                      uint2* __restrict__ W8,
                                                      float* __restrict__ scale_out,
                                                      int32_t* __restrict__ status) {
  __shared__ uint32_t wmax[256 / kWave];
  uint32_t amax = 0;
  for (int i = threadIdx.x; i < npart; i += 256) amax = max(amax, (uint32_t)part[kAmaxX + i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const bool finite = (amax >> 7) < 255;  // bf16 magnitude bits: exponent field all ones
  const float s_w = amax == 0 || !finite ? 1.f : bf16_to_f32((bf16_t)amax) / 448.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *scale_out = s_w;
    if (status) *status = finite ? 0 : kDevScaleRange;
  }
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
    const uint4 q = W[i];
    uint2 o;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cache_quotient(bf16_lo(q.x), s_w),
                                            cache_quotient(bf16_hi(q.x), s_w), 0, false);
    o.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cache_quotient(bf16_lo(q.y), s_w),
                                                    cache_quotient(bf16_hi(q.y), s_w), w, true);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cache_quotient(bf16_lo(q.z), s_w),
                                        cache_quotient(bf16_hi(q.z), s_w), 0, false);
    o.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cache_quotient(bf16_lo(q.w), s_w),
                                                    cache_quotient(bf16_hi(q.w), s_w), w, true);
    W8[i] = o;
  }
}

hipError_t launch_refresh_e4m3(const void* W, int64_t n, void* W8, float* scale_out,
                               int32_t* status, int32_t* part, hipStream_t s) {
  const int64_t nvec = n / 8;
  const int parts = amax_block_count(nvec);
  hipLaunchKernelGGL(k_amax_w, dim3(parts), dim3(kBuildThreads), 0, s, static_cast<const uint4*>(W),
                     nvec, part);
  const int64_t want = (nvec + 255) / 256;
  const int grid = (int)(want < 2048 ? (want > 0 ? want : 1) : 2048);
  hipLaunchKernelGGL(k_refresh_e4m3, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(W),
                     nvec, part, parts, static_cast<uint2*>(W8), scale_out, status);
  return hipGetLastError();
}

}  // namespace sce
