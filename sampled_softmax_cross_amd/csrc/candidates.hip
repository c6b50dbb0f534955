// Candidate-set construction on the device ("sampled_softmax.py",
// CandidateBuilder.build and CandidateBuilder._negatives):
//   mark targets -> count distinct -> walk the stride window for negatives (or the
//   page's fallback) -> ascending C and the class -> position map -> remap labels.
//
// The page builds C on the host with numpy; here it is two kernels on the caller's
// stream, so the step needs no host round trip:
//  * k_cand: one 1024-lane workgroup with the candidate bitmap in LDS does every
//    inherently sequential part (marking, the ordered window walk, the fallback, the
//    ascending compaction into C) and clears the step's counters. It leaves the final
//    bitmap and per-word prefix counts in global memory: a class's position is the
//    count before its word plus the set bits below it in the word, so nothing V-sized
//    is written by the one workgroup;
//  * k_remap_gather: a grid kernel whose blocks remap every label to its position and
//    count N, copy the candidates' rows of W (the gather, see gather_scatter.hip for
//    the copy itself), clear the dense gradient's rows outside C and, when asked,
//    write the class -> position map.
#include "common.h"
#include "kernels.h"

namespace sce {

__device__ __forceinline__ uint32_t valid_bits(int w, int V) {
  const int rem = V - w * 32;
  return rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
}

// Position of class c in C from the final bitmap and per-word prefix counts (-1: c is
// not a candidate).
__device__ __forceinline__ int class_pos(const uint32_t* __restrict__ bits,
                                         const int32_t* __restrict__ wpre, int c) {
  // both words are loaded before either is used (no load waits alone behind a branch)
  const uint32_t m = bits[c >> 5];
  const int pre = wpre[c >> 5];
  const int b = c & 31;
  return ((m >> b) & 1u) ? pre + __popc(m & ((1u << b) - 1u)) : -1;
}

// Dynamic LDS: 2 * ceil(V/32) words when mark_lds (V <= SCE_MAX_V_SAMPLED), else none.
// P == 0 (full softmax): only the distinct count (when the bitmap fits) and the
// label range check; C and the bitmap are not built. P > 0: C, and bits / wpre
// (ceil(V/32) words each: the candidate bitmap and the number of candidates before
// each word).
__global__ __launch_bounds__(kBuildThreads) void k_cand(const int64_t* __restrict__ targets,
                                                        const int64_t* __restrict__ prefix,
                                                        int T, int V, int P, int stride, int off,
                                                        bool mark_lds, int32_t* __restrict__ C,
                                                        uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ wpre,
                                                        int32_t* __restrict__ counters,
                                                        const uint4* __restrict__ amax_x,
                                                        int64_t amax_nvec, int x_parts,
                                                        const uint4* __restrict__ amax_w,
                                                        int64_t amax_w_nvec) {
  // Blocks past the first: the e4m3 step's max|x| (x_parts blocks, one partial each),
  // then, when the step encodes bf16 weights itself, max|W| (partials at kAmaxW). They
  // need nothing from the build and run beside it on the otherwise idle chip.
  if (blockIdx.x > 0) {
    const int b = (int)blockIdx.x - 1;
    if (b < x_parts)
      amax_bf16_block<kAmaxLoadsBuild>(amax_x, amax_nvec, b, x_parts, counters);
    else
      amax_bf16_block<kAmaxLoadsBuild>(amax_w, amax_w_nvec, b - x_parts, (int)gridDim.x - 1 - x_parts,
                      counters + (kAmaxW - kAmaxX));
    return;
  }
  extern __shared__ uint32_t lds_words[];
  __shared__ int scratch[kBuildThreads / kWave + 1];
  const int W = (V + 31) >> 5;
  uint32_t* mark = lds_words;     // candidate bitmap
  uint32_t* aux = lds_words + W;  // window picks, then per-word prefix counts
  const int tid = threadIdx.x;
  const int nt = blockDim.x;

  if (tid < kNumCounters) counters[tid] = 0;
  if (mark_lds)
    for (int w = tid; w < W; w += nt) {
      mark[w] = 0;
      aux[w] = 0;
    }
  __syncthreads();

  // 1. Mark every class that is a target; range-check targets and prefix targets.
  //    Each lane loads kMarkLoads labels before it uses any, so one workgroup keeps
  //    enough loads in flight to stream the label arrays.
  constexpr int kMarkLoads = 8;
  int bad = 0;
  for (int t0 = tid; t0 < T; t0 += nt * kMarkLoads) {
    int64_t y[kMarkLoads], q[kMarkLoads];
#pragma unroll
    for (int j = 0; j < kMarkLoads; ++j) {
      const int t = t0 + j * nt;
      y[j] = t < T ? targets[t] : -1;
      q[j] = (prefix != nullptr && t < T) ? prefix[t] : -1;
    }
#pragma unroll
    for (int j = 0; j < kMarkLoads; ++j) {
      if (y[j] < -1 || y[j] >= V) {
        bad = 1;
      } else if (y[j] >= 0 && mark_lds) {
        atomicOr(&mark[y[j] >> 5], 1u << (y[j] & 31));
      }
      if (q[j] < -1 || q[j] >= V) bad = 1;
    }
  }
  __syncthreads();
  int cnt = 0;
  if (mark_lds)
    for (int w = tid; w < W; w += nt) cnt += __popc(mark[w]);
  // One block sum carries both: the distinct count (below 2^20: V <= 131072 when the
  // bitmap is in LDS, else 0) and, above it, the lanes that met a bad label (<= 1024).
  const int packed = block_sum_int(cnt + (bad << 20), scratch);  // (contains barriers)
  const int distinct = packed & ((1 << 20) - 1);
  const int any_bad = packed >> 20;
  if (P == 0) {
    if (tid == 0) {
      counters[kStatus] = any_bad ? kDevLabelRange : 0;
      counters[kDistinct] = mark_lds ? distinct : -1;
      counters[kNextOffset] = off;
    }
    return;
  }
  int status = any_bad ? kDevLabelRange : 0;
  const int need = P - distinct;
  int next_off = off;
  if (need < 0) {
    // The page asserts this never happens. Flag it and leave a harmless map
    // (C = [0, P)) so that every later kernel stays in bounds.
    status |= kDevTooManyTargets;
    for (int w = tid; w < W; w += nt) {
      const int lo = w * 32;
      mark[w] = P >= lo + 32 ? 0xffffffffu : (P > lo ? (1u << (P - lo)) - 1u : 0u);
    }
  } else if (need > 0) {
    const int draw = min(V, (17 * need) / 10 + 256);  // == floor(1.7 * need) + 256
    next_off = (int)(((int64_t)off + draw) % V);
    // 2. Walk window positions i = 0 .. draw-1 (class ((off+i) mod V) * stride mod V)
    //    in order; the first `need` free classes become negatives. Each lane takes
    //    kWalk consecutive positions; a block scan orders the lanes.
    constexpr int kWalk = 4;
    int seen = 0;  // free classes met so far (block-uniform)
    for (int base = 0; base < draw && seen < need; base += nt * kWalk) {
      const int i0 = base + tid * kWalk;
      int cls[kWalk];
      uint32_t freemask = 0;
      int c = 0;
      if (i0 < draw) c = (int)(((int64_t)((off + i0) % V) * stride) % V);
#pragma unroll
      for (int j = 0; j < kWalk; ++j) {
        cls[j] = c;
        if (i0 + j < draw && !((mark[c >> 5] >> (c & 31)) & 1u)) freemask |= 1u << j;
        c += stride;
        if (c >= V) c -= V;
      }
      int total;
      int rank = block_exclusive_scan(__popc(freemask), scratch, &total) + seen;
#pragma unroll
      for (int j = 0; j < kWalk; ++j) {
        if ((freemask >> j) & 1u) {
          if (rank < need) atomicOr(&aux[cls[j] >> 5], 1u << (cls[j] & 31));
          ++rank;
        }
      }
      seen += total;
    }
    __syncthreads();
    const int wpt = (W + nt - 1) / nt;  // contiguous words per lane keeps class order
    const int w0 = min(W, tid * wpt), w1 = min(W, w0 + wpt);
    if (seen >= need) {
      for (int w = tid; w < W; w += nt) mark[w] |= aux[w];
    } else {
      // 3. Fallback: every step-th free class in ascending order, first `need`.
      const int step = max(1, (V - distinct) / need);
      int nfree = 0;
      for (int w = w0; w < w1; ++w) nfree += __popc(~mark[w] & valid_bits(w, V));
      int total;
      int r = block_exclusive_scan(nfree, scratch, &total);
      for (int w = w0; w < w1; ++w) {
        uint32_t fm = ~mark[w] & valid_bits(w, V);
        uint32_t sel = 0;
        while (fm) {
          const int b = __ffs(fm) - 1;
          fm &= fm - 1;
          if (r % step == 0 && r / step < need) sel |= 1u << b;
          ++r;
        }
        mark[w] |= sel;
      }
    }
  }
  __syncthreads();

  // 4. Ascending compaction: per-word prefix counts, C, then the bitmap and the prefix
  //    counts go out for the grid kernels. C: with few candidates per word, each lane
  //    walks the set bits of its contiguous words (a contiguous stretch of C); with
  //    many, every lane takes every nt-th class (a fixed trip count). Measured at
  //    V = 50304: 18.6 vs 20.4 us for the build and remap at P = 10240, 41.7 vs 35.4 us
  //    at P = 24576 with prefix targets.
  const bool sparse = 10 * (int64_t)P <= 3 * (int64_t)V;
  {
    const int wpt = (W + nt - 1) / nt;
    const int w0 = min(W, tid * wpt), w1 = min(W, w0 + wpt);
    int pc = 0;
    for (int w = w0; w < w1; ++w) pc += __popc(mark[w]);
    int total;
    int r = block_exclusive_scan(pc, scratch, &total);
    for (int w = w0; w < w1; ++w) {
      aux[w] = (uint32_t)r;
      uint32_t m = mark[w];
      if (sparse) {
        while (m) {
          const int b = __ffs(m) - 1;
          m &= m - 1;
          C[r++] = w * 32 + b;
        }
      } else {
        r += __popc(m);
      }
    }
  }
  __syncthreads();
  if (!sparse) {
#pragma unroll 4
    for (int c = tid; c < V; c += nt) {
      const uint32_t m = mark[c >> 5];
      const int b = c & 31;
      if ((m >> b) & 1u) C[(int)aux[c >> 5] + __popc(m & ((1u << b) - 1u))] = c;
    }
  }
  for (int w = tid; w < W; w += nt) {
    bits[w] = mark[w];
    wpre[w] = (int)aux[w];
  }
  if (tid == 0) {
    counters[kStatus] = status;
    counters[kDistinct] = distinct;
    counters[kNextOffset] = next_off;
  }
}

// Blocks [0, remap_blocks): labels -> positions in C (identity when P == 0), count N.
// The next gather_blocks: the row gather W_C = W[C] (none when P == 0), or with WT
// (bf16) tiles that gather and transpose: W_C and WT = W_C^T from one read. The next
// zero_blocks: the rows of the dense gradient outside C set to zero (written here,
// while the memory system is otherwise idle, rather than beside the candidate rows at
// the end of the step). The rest: vocab_pos[c] = position of c in C, or -1.
__global__ __launch_bounds__(256) void k_remap_gather(
    const int64_t* __restrict__ targets, const int64_t* __restrict__ prefix, int T, int V, int P,
    const uint32_t* __restrict__ bits, const int32_t* __restrict__ wpre,
    int32_t* __restrict__ target_pos, int32_t* __restrict__ prefix_pos,
    int32_t* __restrict__ counters, int remap_blocks, const uint4* __restrict__ W,
    const int32_t* __restrict__ C, int row_vecs, uint4* __restrict__ WC, int wc_vecs,
    int gather_blocks, uint4* __restrict__ dW, int dw_vecs, int zero_blocks,
    int32_t* __restrict__ vocab_pos, uint16_t* __restrict__ WT, int64_t ldt, int tr_x,
    const int32_t* __restrict__ tpos_in, const int32_t* __restrict__ ppos_in, int enc_parts,
    float* __restrict__ enc_slot, float* __restrict__ enc_out) {
  const int b = (int)blockIdx.x;
  if (b >= remap_blocks + gather_blocks + zero_blocks) {
    const int c = (b - remap_blocks - gather_blocks - zero_blocks) * 256 + (int)threadIdx.x;
    if (c < V) vocab_pos[c] = class_pos(bits, wpre, c);
    return;
  }
  if (b >= remap_blocks + gather_blocks) {
    zero_rows_block(b - remap_blocks - gather_blocks, bits, V, dw_vecs, dW);
    return;
  }
  if ((int)blockIdx.x >= remap_blocks) {
    const int g = (int)blockIdx.x - remap_blocks;
    if (enc_parts > 0) {
      // the gather with encoding: s_w from the max|W| partials (each block forms it; the
      // first publishes it), then the codes of the bf16 rows W[C] (every row at P == 0)
      __shared__ uint32_t wmax[256 / kWave];
      uint32_t amax = 0;
      for (int i = threadIdx.x; i < enc_parts; i += 256)
        amax = max(amax, (uint32_t)counters[kAmaxW + i]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, kWave));
      if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = amax;
      __syncthreads();
      amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
      const bool finite = (amax >> 7) < 255;  // bf16 magnitude bits: exponent all ones
      const float s_w = amax == 0 || !finite ? 1.f : bf16_to_f32((bf16_t)amax) / 448.f;
      if (g == 0 && threadIdx.x == 0) {
        *enc_slot = s_w;
        if (enc_out) *enc_out = s_w;
        if (!finite) atomicOr(&counters[kStatus], kDevScaleRange);
      }
      gather_encode_block(g, W, P > 0 ? C : nullptr, P > 0 ? P : V, row_vecs,
                          reinterpret_cast<uint8_t*>(WC), (int64_t)wc_vecs * 16, s_w);
      return;
    }
    if (WT)
      transpose_tile<uint16_t>(g % tr_x, g / tr_x, reinterpret_cast<const uint16_t*>(W),
                               (int64_t)row_vecs * 8, C, P, row_vecs * 8, WT, ldt,
                               reinterpret_cast<uint16_t*>(WC), (int64_t)wc_vecs * 8);
    else
      gather_rows_block(g, W, C, P, row_vecs, WC, wc_vecs);
    return;
  }
  __shared__ int scratch[256 / kWave + 1];
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  int n = 0;
  if (t < T && tpos_in != nullptr) {
    // Positions given (a candidate set built beforehand): copied, with a position outside
    // [-1, P) flagged and replaced by -1.
    int tp = tpos_in[t];
    int pp = ppos_in != nullptr ? ppos_in[t] : -1;
    const bool bad = tp < -1 || tp >= P || pp < -1 || pp >= P;
    if (tp < -1 || tp >= P) tp = -1;
    if (pp < -1 || pp >= P) pp = -1;
    if (bad) atomicOr(&counters[kStatus], kDevLabelRange);
    target_pos[t] = tp;
    prefix_pos[t] = pp;
    n += (tp >= 0) + (pp >= 0);
  } else if (t < T) {
    // Both labels, then (sampled) their bitmap words, each set of loads issued before
    // any of them is used; a label outside [0, V) looks up class 0 and is dropped.
    const int64_t y = targets[t];
    const int64_t p = prefix != nullptr ? prefix[t] : -1;
    const bool yv = y >= 0 && y < V, pv = p >= 0 && p < V;
    int tp = yv ? (int)y : -1, pp = pv ? (int)p : -1;
    if (P > 0) {
      const int tq = class_pos(bits, wpre, yv ? (int)y : 0);
      const int pq = prefix != nullptr ? class_pos(bits, wpre, pv ? (int)p : 0) : -1;
      tp = yv ? tq : -1;
      pp = pv ? pq : -1;
    }
    target_pos[t] = tp;
    prefix_pos[t] = pp;
    n += (tp >= 0) + (pp >= 0);
  }
  const int s = block_sum_int(n, scratch);
  if (threadIdx.x == 0 && s) atomicAdd(&counters[kNumLabels], s);
}

// A candidate set built beforehand (P > 0): one workgroup clears the step's counters,
// copies C to the step's own array with every class that is outside [0, V) or not above
// its predecessor flagged (SCE_DEV_LABEL_RANGE) and replaced by class 0 (so every later
// access stays in bounds), leaves the candidate bitmap for the launch that clears dW's
// other rows, and takes the distinct count, next offset and device bits from the build's
// aux when given (else -1, -1, 0).
__global__ __launch_bounds__(kBuildThreads) void k_cand_prebuilt(
    const int32_t* __restrict__ C_in, int V, int P, const int64_t* __restrict__ build_aux,
    int32_t* __restrict__ counters, int32_t* __restrict__ C, uint32_t* __restrict__ bits,
    const uint4* __restrict__ amax_x, int64_t amax_nvec) {
  // Blocks past the first: the e4m3 step's max|x| partials, as beside the device build.
  if (blockIdx.x > 0) {
    amax_bf16_block<kAmaxLoadsBuild>(amax_x, amax_nvec, (int)blockIdx.x - 1, (int)gridDim.x - 1, counters);
    return;
  }
  extern __shared__ uint32_t mark[];
  __shared__ int scratch[kBuildThreads / kWave + 1];
  const int W = (V + 31) >> 5;
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid < kNumCounters) counters[tid] = 0;
  for (int w = tid; w < W; w += nt) mark[w] = 0;
  __syncthreads();
  int bad = 0;
  for (int i = tid; i < P; i += nt) {
    const int c = C_in[i];
    const int prev = i > 0 ? C_in[i - 1] : -1;
    const bool ok = c >= 0 && c < V && c > prev;
    bad |= !ok;
    C[i] = ok ? c : 0;
    if (ok) atomicOr(&mark[c >> 5], 1u << (c & 31));
  }
  const int any_bad = block_sum_int(bad, scratch);  // (contains barriers)
  for (int w = tid; w < W; w += nt) bits[w] = mark[w];
  if (tid == 0) {
    counters[kStatus] = (any_bad ? kDevLabelRange : 0) | (build_aux ? (int)build_aux[3] : 0);
    counters[kDistinct] = build_aux ? (int)build_aux[0] : -1;
    counters[kNextOffset] = build_aux ? (int)build_aux[2] : -1;
  }
}

__global__ void k_write_aux(const int32_t* __restrict__ counters, int64_t* __restrict__ aux) {
  if (threadIdx.x == 0) {
    aux[0] = counters[kDistinct];
    aux[1] = counters[kNumLabels];
    aux[2] = counters[kNextOffset];
    aux[3] = counters[kStatus];
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_candidates(const int64_t* targets, const int64_t* prefix, int T, int V, int P,
                             int stride, int off, int32_t* counters, int32_t* C, uint32_t* bits,
                             int32_t* wpre, int32_t* vocab_pos, int32_t* target_pos,
                             int32_t* prefix_pos, const void* W, int row_bytes, void* WC,
                             int wc_row_bytes, void* dW, int dw_row_bytes, hipStream_t s,
                             const void* amax_x, int64_t amax_n, int* amax_parts, void* WT,
                             int64_t ldt, CacheEncode* enc) {
  const bool mark_lds = V <= kMaxBitmapClasses;
  const size_t lds = mark_lds ? (size_t)2 * ((V + 31) / 32) * sizeof(uint32_t) : 0;
  const int agrid = amax_n >= 0 ? amax_block_count<kAmaxLoadsBuild>(amax_n / 8) : 0;
  if (amax_parts) *amax_parts = agrid;
  // with enc: W holds bf16 rows of row_bytes; its max|W| partials come from more blocks
  const int64_t w_nvec = enc ? (int64_t)V * (row_bytes / 16) : 0;
  const int wgrid = enc ? amax_block_count<kAmaxLoadsBuild>(w_nvec) : 0;
  if (enc) {
    if (W == nullptr || WT != nullptr || enc->scale_slot == nullptr) return hipErrorInvalidValue;
    enc->w_parts = wgrid;
  }
  hipLaunchKernelGGL(k_cand, dim3(1 + agrid + wgrid), dim3(kBuildThreads), lds, s, targets, prefix,
                     T, V, P, stride, off, mark_lds, C, bits, wpre, counters,
                     static_cast<const uint4*>(amax_x), amax_n / 8, agrid,
                     static_cast<const uint4*>(enc ? W : nullptr), w_nvec);
  const int remap_blocks = (T + 255) / 256;
  // with WT: gather-and-transpose tiles, kTrTile rows of W_C by kTrTile of its columns
  const bool tr = WT != nullptr && W != nullptr && P > 0;
  const int tr_x = tr ? (int)((ldt + kTrTile - 1) / kTrTile) : 1;
  const int gather_blocks =
      enc ? gather_block_count(P > 0 ? P : V, row_bytes / 16)
      : tr ? tr_x * ((row_bytes / 2 + kTrTile - 1) / kTrTile)
           : ((W != nullptr && P > 0) ? gather_block_count(P, row_bytes / 16) : 0);
  const int zero_blocks = (dW != nullptr && P > 0) ? zero_block_count(V, dw_row_bytes / 16) : 0;
  const int map_blocks = (vocab_pos != nullptr && P > 0) ? (V + 255) / 256 : 0;
  const int grid = remap_blocks + gather_blocks + zero_blocks + map_blocks;
  if (grid > 0)
    hipLaunchKernelGGL(k_remap_gather, dim3(grid), dim3(256), 0, s, targets, prefix, T, V, P, bits,
                       wpre, target_pos, prefix_pos, counters, remap_blocks,
                       reinterpret_cast<const uint4*>(W), C, row_bytes / 16,
                       reinterpret_cast<uint4*>(WC), wc_row_bytes / 16, gather_blocks,
                       reinterpret_cast<uint4*>(dW), dw_row_bytes / 16, zero_blocks, vocab_pos,
                       static_cast<uint16_t*>(tr ? WT : nullptr), ldt, tr_x, nullptr, nullptr,
                       enc ? enc->w_parts : 0, enc ? enc->scale_slot : nullptr,
                       enc ? enc->scale_out : nullptr);
  return hipGetLastError();
}

hipError_t launch_candidates_prebuilt(const int32_t* C_in, const int32_t* tpos_in,
                                      const int32_t* ppos_in, const int64_t* build_aux, int T,
                                      int V, int P, int32_t* counters, int32_t* C, uint32_t* bits,
                                      int32_t* target_pos, int32_t* prefix_pos, const void* W,
                                      int row_bytes, void* WC, int wc_row_bytes, void* dW,
                                      int dw_row_bytes, void* WT, int64_t ldt, hipStream_t s,
                                      const void* amax_x, int64_t amax_n, int* amax_parts) {
  if (P < 1 || V > kMaxBitmapClasses) return hipErrorInvalidValue;
  const size_t lds = (size_t)((V + 31) / 32) * sizeof(uint32_t);
  const int agrid = amax_n >= 0 ? amax_block_count<kAmaxLoadsBuild>(amax_n / 8) : 0;
  if (amax_parts) *amax_parts = agrid;
  hipLaunchKernelGGL(k_cand_prebuilt, dim3(1 + agrid), dim3(kBuildThreads), lds, s, C_in, V, P,
                     build_aux, counters, C, bits, static_cast<const uint4*>(amax_x), amax_n / 8);
  // the remap launch in its positions mode: the same gather (with the transpose), zero rows
  // and label counting as after a build, with the positions copied instead of derived
  const int remap_blocks = (T + 255) / 256;
  const bool tr = WT != nullptr && W != nullptr;
  const int tr_x = tr ? (int)((ldt + kTrTile - 1) / kTrTile) : 1;
  const int gather_blocks = tr ? tr_x * ((row_bytes / 2 + kTrTile - 1) / kTrTile)
                               : (W != nullptr ? gather_block_count(P, row_bytes / 16) : 0);
  const int zero_blocks = dW != nullptr ? zero_block_count(V, dw_row_bytes / 16) : 0;
  const int grid = remap_blocks + gather_blocks + zero_blocks;
  if (grid > 0)
    hipLaunchKernelGGL(k_remap_gather, dim3(grid), dim3(256), 0, s, nullptr, nullptr, T, V, P,
                       bits, nullptr, target_pos, prefix_pos, counters, remap_blocks,
                       reinterpret_cast<const uint4*>(W), C, row_bytes / 16,
                       reinterpret_cast<uint4*>(WC), wc_row_bytes / 16, gather_blocks,
                       reinterpret_cast<uint4*>(dW), dw_row_bytes / 16, zero_blocks, nullptr,
                       static_cast<uint16_t*>(tr ? WT : nullptr), ldt, tr_x, tpos_in,
                       T > 0 ? ppos_in : nullptr, 0, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_write_aux(const int32_t* counters, int64_t* aux, hipStream_t s) {
  hipLaunchKernelGGL(k_write_aux, dim3(1), dim3(64), 0, s, counters, aux);
  return hipGetLastError();
}

}  // namespace sce
