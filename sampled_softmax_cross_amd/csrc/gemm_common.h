// Pieces shared by the GEMM kernels (gfx950): operand tiles, buffer loads, the
// XCD-aware tile order and the register epilogue.
#pragma once

#include "common.h"
#include "kernels.h"

namespace sce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kNumXcd = 8;
constexpr int kGroupM = 8;

// Index (in 16-byte units) of chunk `ch` of operand-tile row `row`.
__device__ __forceinline__ int lds_index(int row, int ch) {
  return row * 8 + (ch ^ ((row ^ (row >> 3)) & 7));
}

template <typename TIn>
struct Elem {
  static constexpr int kSize = sizeof(TIn);
  static constexpr int kVec = 16 / kSize;    // elements per 16-byte vector
  static constexpr int kTileK = 128 / kSize; // k elements per LDS row
};

// Raw buffer loads: an offset at or beyond num_records reads zeros, which clips the
// tile edges without branches. Offsets are relative to a per-tile base address.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kOOB = 0x7ffffff0;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kOOB, 0x00020000);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for an LDS ring filled by buffer_load ... lds: this wave's LDS reads
// complete (lgkmcnt 0), then s_barrier. Each wave waits for its own loads into the ring
// (vmcnt) before calling it. A fenced __syncthreads would also wait for every
// outstanding load and store of the wave (vmcnt 0: the loads write LDS), which empties
// a ring meant to keep stages in flight across the barrier. The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

enum OutMode { kOutBF16 = 0, kOutF32 = 1, kOutF32Split = 2, kOutDW = 3 };



// Output tile of workgroup `bid` among nby x nbx tiles: XCD-contiguous, grouped.
__device__ __forceinline__ void tile_of(int bid, int nby, int nbx, int& tm, int& tn) {
  const int total = nby * nbx;
  const int q = total / kNumXcd, rem = total % kNumXcd;
  const int x = bid % kNumXcd, i = bid / kNumXcd;
  const int lid = x < rem ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
  const int per_group = kGroupM * nbx;
  const int g = lid / per_group;
  const int first = g * kGroupM;
  const int gsize = min(nby - first, kGroupM);
  const int in = lid - g * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

// Rows per group of the tile order for outputs of many column tiles. Within a group the
// order walks all nbx column tiles for `g` rows, so a B (column) tile is reused after the
// XCD has written g * nbx output tiles; chip-wide that is g * nbx * tile_bytes * 8 bytes of
// output streaming through the 256 MB MALL. The largest g in {8, 4, 2} that keeps this
// under the MALL's size lets the reused B tiles still hit there; when none does, 8 (the
// best L2 reuse of the A rows). Measured on the logits products: 5-18% faster than a
// fixed 8 at P = 14336 and 24576 (T = 49152), equal elsewhere.
__device__ __forceinline__ int group_rows(int nbx, int64_t tile_bytes) {
  constexpr int64_t kMall = 256ll << 20;
  for (int g = 8; g >= 2; g >>= 1)
    if ((int64_t)g * nbx * tile_bytes * kNumXcd <= kMall) return g;
  return 8;
}

// Unit u of `total` renumbered XCD-contiguously: workgroup ids are dealt round-robin
// over the XCDs, so u % kNumXcd is the unit's XCD (any constant shift of u keeps the
// XCD groups intact); the XCD's units get consecutive numbers.
__device__ __forceinline__ int xcd_order(int u, int total) {
  const int q = total / kNumXcd, rem = total % kNumXcd;
  const int x = u % kNumXcd, i = u / kNumXcd;
  return x < rem ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
}

// Tile and k-range of unit u among nby x nbx tiles x `splits` k-ranges. Units are
// renumbered XCD-contiguously (workgroup ids are dealt round-robin over the XCDs) with the
// k-range outermost, so each XCD works on one k-range. Within a k-range, tiles go
// row-major when there are at most 4 column tiles (every column tile of a row shares the
// row's A block, and they land on the same XCD), otherwise in groups of `gm` rows.
__device__ __forceinline__ void unit_of(int u, int nby, int nbx, int splits, int gm, int& tm,
                                        int& tn, int& split) {
  const int ntiles = nby * nbx;
  const int lid = xcd_order(u, ntiles * splits);
  split = lid / ntiles;
  const int t = lid - split * ntiles;
  if (nbx <= 4) {
    tm = t / nbx;
    tn = t - tm * nbx;
    return;
  }
  const int per_group = gm * nbx;
  const int g = t / per_group;
  const int first = g * gm;
  const int gsize = min(nby - first, gm);
  const int in = t - g * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

// Compute units of the current device (cached per device; 256 when unknown).
inline int cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

// Store the accumulators of one wave. Accumulator r of lane l in block (i, j) is
// output row rbase + i*32 (rbase includes l % 32), output column
// cbase + j*32 + 8*(r/4) + 4*(l/32) + r%4 (the MFMA is issued with the B-tile
// fragment first, so each block is the transposed 32 x 32 output). Columns are
// stored up to N rounded up to 8: every ldc is a multiple of 8 and at least that,
// and padding columns receive zeros.
template <int OUT, int TM, int TN>
__device__ __forceinline__ void store_acc(f32x16_t (&acc)[TM][TN], void* __restrict__ Cout, int64_t ldc,
                                          int64_t M, int64_t N, int64_t rbase, int64_t cbase,
                                          int half, int64_t split_offset) {
  const int64_t ncols = (N + 7) / 8 * 8;
  if constexpr (OUT == kOutBF16) {
    // Pack to bf16 (4 columns = 2 dwords per register group g), then swap groups
    // between lane halves so that the low half holds columns 8g..8g+7 of even g and
    // the high half those of odd g: 16 contiguous bytes per lane and group pair.
    bf16_t* out = static_cast<bf16_t*>(Cout);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t row = rbase + i * 32;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {  // register groups (2gp, 2gp+1)
          const int g0 = 4 * (2 * gp), g1 = 4 * (2 * gp + 1);
          uint32_t e0 = pack_bf16x2(acc[i][j][g0 + 0], acc[i][j][g0 + 1]);
          uint32_t e1 = pack_bf16x2(acc[i][j][g0 + 2], acc[i][j][g0 + 3]);
          uint32_t o0 = pack_bf16x2(acc[i][j][g1 + 0], acc[i][j][g1 + 1]);
          uint32_t o1 = pack_bf16x2(acc[i][j][g1 + 2], acc[i][j][g1 + 3]);
          // lanes 32+l <-> l: the high half's even group meets the low half's odd group
          const auto s0 = __builtin_amdgcn_permlane32_swap(e0, o0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(e1, o1, false, false);
          e0 = s0[0]; o0 = s0[1];
          e1 = s1[0]; o1 = s1[1];
          // low half: columns 8*(2gp) .. +7 = {e, o};  high half: 8*(2gp+1) .. +7 = {e, o}
          const int64_t col = cbase + j * 32 + 8 * (2 * gp + half);
          if (row < M && col < ncols)
            *reinterpret_cast<uint4*>(out + row * ldc + col) = make_uint4(e0, e1, o0, o1);
        }
      }
    }
  } else {
    float* out = static_cast<float*>(Cout) + split_offset;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t row = rbase + i * 32;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = cbase + j * 32 + 8 * g + 4 * half;
          if (row < M && col < ncols)
            *reinterpret_cast<float4*>(out + row * ldc + col) =
                make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        }
    }
  }
}

// bf16 output of one wave into rows picked by `rowmap` (output row r goes to row
// rowmap[r], or r when rowmap is null): the layout of store_acc's bf16 case, with the
// destination row looked up once per 32-row block (rows >= M are not stored).
template <int TM, int TN>
__device__ __forceinline__ void store_acc_rows_bf16(f32x16_t (&acc)[TM][TN], void* __restrict__ Cout,
                                                    int64_t ldc, const int32_t* __restrict__ rowmap,
                                                    int64_t M, int64_t N, int64_t rbase,
                                                    int64_t cbase, int half) {
  const int64_t ncols = (N + 7) / 8 * 8;
  bf16_t* out = static_cast<bf16_t*>(Cout);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = rbase + i * 32;
    const int64_t dst = row < M ? (rowmap ? (int64_t)rowmap[row] : row) : 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const int g0 = 4 * (2 * gp), g1 = 4 * (2 * gp + 1);
        uint32_t e0 = pack_bf16x2(acc[i][j][g0 + 0], acc[i][j][g0 + 1]);
        uint32_t e1 = pack_bf16x2(acc[i][j][g0 + 2], acc[i][j][g0 + 3]);
        uint32_t o0 = pack_bf16x2(acc[i][j][g1 + 0], acc[i][j][g1 + 1]);
        uint32_t o1 = pack_bf16x2(acc[i][j][g1 + 2], acc[i][j][g1 + 3]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(e0, o0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(e1, o1, false, false);
        e0 = s0[0]; o0 = s0[1];
        e1 = s1[0]; o1 = s1[1];
        const int64_t col = cbase + j * 32 + 8 * (2 * gp + half);
        if (row < M && col < ncols)
          *reinterpret_cast<uint4*>(out + dst * ldc + col) = make_uint4(e0, e1, o0, o1);
      }
    }
  }
}

// bf16 output of a wave whose slice is 64 columns wide (TN = 2), restaged through
// `stage` (4 KB of LDS owned by the wave) one 32-row block at a time: each lane writes
// its row's four 16-byte pieces (column chunks c = 4j + 2gp + half, placed at chunk
// slot c ^ (row & 7) so that eight lanes of one chunk hit all 32 banks), then reads
// back eight rows of eight chunks per instruction, so that every store instruction
// writes eight whole 128-byte rows instead of 32-byte pieces of 32 rows (the same 16
// stores per lane; the logits product spends less time in its epilogue).
template <int TM, int TN>
__device__ __forceinline__ void store_acc_bf16_lds(f32x16_t (&acc)[TM][TN], void* __restrict__ Cout,
                                                   int64_t ldc, int64_t M, int64_t N, int64_t row0,
                                                   int64_t col0, int lane, uint4* __restrict__ stage) {
  static_assert(TN == 2, "64-column wave slices: eight 16-byte chunks per row");
  bf16_t* out = static_cast<bf16_t*>(Cout);
  const int64_t ncols = (N + 7) / 8 * 8;
  const int l32 = lane & 31, half = lane >> 5;
  const int rr = lane >> 3, cc = lane & 7;  // read-back: row rr of each group of 8, chunk cc
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const int g0 = 4 * (2 * gp), g1 = 4 * (2 * gp + 1);
        uint32_t e0 = pack_bf16x2(acc[i][j][g0 + 0], acc[i][j][g0 + 1]);
        uint32_t e1 = pack_bf16x2(acc[i][j][g0 + 2], acc[i][j][g0 + 3]);
        uint32_t o0 = pack_bf16x2(acc[i][j][g1 + 0], acc[i][j][g1 + 1]);
        uint32_t o1 = pack_bf16x2(acc[i][j][g1 + 2], acc[i][j][g1 + 3]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(e0, o0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(e1, o1, false, false);
        const int c = 4 * j + 2 * gp + half;
        stage[l32 * 8 + (c ^ (l32 & 7))] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
    }
    // the wave's LDS writes complete before any lane reads another lane's row
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + rr;
      v[q] = stage[r * 8 + (cc ^ (r & 7))];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next block's writes
    const int64_t col = col0 + 8 * cc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = row0 + i * 32 + 8 * q + rr;
      if (row < M && col < ncols) *reinterpret_cast<uint4*>(out + row * ldc + col) = v[q];
    }
  }
}

}  // namespace sce
