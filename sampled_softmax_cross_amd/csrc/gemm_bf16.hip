// Multi-stage MFMA GEMM for gfx950 (the logits, dX and dW products of the step), for
// bf16 operands (EB = 2 bytes per element) and OCP e4m3 operands (EB = 1).
//
// Every operand tile travels global -> LDS by buffer_load ... lds (no VGPR staging,
// no ds_write), through an NS-deep ring of LDS stages of SK k each, so a tile is
// requested NS-1 stage-times before the MFMAs need it and the load latency of a busy
// memory system stays hidden behind the matrix cores.
//
// Operand layouts in LDS (16-byte chunks):
//  * r-major (element (r, k) at P[r * ld + k], k contiguous): rows of SK k (64 or
//    128 B), the chunks of a row XOR-swizzled by ((row >> 1) ^ (row >> 3)) & 3 (64-byte
//    rows) or (row >> 1) & 7 (128-byte rows). A lane's fragment is 16 (bf16) or 32
//    (e4m3) consecutive bytes of one row: one or two ds_read_b128. With 128-byte rows
//    every row of a stage is one whole line of the operand, which halves the cache
//    requests per byte against 64-byte rows.
//  * k-major (element (r, k) at P[k * ld + r]): the tile is kept as it is in memory,
//    SK rows of k, each R elements wide. bf16: chunks XOR-swizzled by 4 * (k & 3) (rows
//    of a multiple of 256 bytes) or 4 * ((k >> 1) & 1) (384-byte rows); fragments are
//    read with ds_read_b64_tr_b16: within each 16-lane group, lane j receives element i
//    from the address supplied by lane 4i + j/4 (at element offset j % 4), so lanes
//    that point at rows k..k+3 and 4-column groups assemble 8-k fragments of single
//    columns. e4m3: chunks XOR-swizzled by 2 * (k & 7) (rows of a multiple of 256
//    bytes), k & 7 (128-byte rows) or (k >> 1) & 3 (192-byte rows);
//    ds_read_b64_tr_b8 gives lane j byte i from the
//    address of lane 2i + j/8 (at byte offset j % 8): lanes pointing at rows k..k+7 and
//    8-column groups assemble 8-k pieces of single columns, four of which make a
//    32-k fragment.
// The swizzles spread a fragment read over all LDS banks; the DMA fill picks, for each
// lane, the global chunk that belongs at its (linear) LDS position.
//
// The MFMA (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// scales for e4m3) takes the B-tile fragment first, which makes every accumulator
// block the transposed output and lets the epilogue write 16-byte vectors straight
// from registers (see store_acc). Lane l holds k = kgroup * (l / 32) + [0, kgroup) of
// its row or column in both operands (8 for bf16, 32 for e4m3).
#include "gemm_common.h"

namespace sce {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Per element size: the fragment a lane holds for one MFMA and the k one MFMA covers.
template <int EB>
struct MfmaElem;
template <>
struct MfmaElem<2> {
  using frag_t = bf16x8_t;
  static constexpr int kMfmaK = 16;
};
template <>
struct MfmaElem<1> {
  using frag_t = i32x8_t;
  static constexpr int kMfmaK = 64;
};

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt at their maxima (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS chunk (16 B) holding chunk `ch` of r-major row `row` (CPR chunks per row).
template <int CPR>
__device__ __forceinline__ int rm_swizzle(int row) {
  if constexpr (CPR == 4) return ((row >> 1) ^ (row >> 3)) & 3;
  else return (row >> 1) & 7;
}
template <int CPR>
__device__ __forceinline__ int rm_index(int row, int ch) {
  return row * CPR + (ch ^ rm_swizzle<CPR>(row));
}
// k-major chunk swizzle for rows of RB bytes: the rows one transposing read touches
// land on distinct bank groups. bf16 reads touch rows k..k+3 with 8 bytes each per
// lane quad: rows of a multiple of 256 bytes start on the same banks, so they shift by
// 4 * (k & 3) chunks; 384-byte rows alternate between two bank offsets, so rows k and
// k + 2 shift by 4 chunks. e4m3 reads touch rows k..k+7 and two adjacent chunks, 16
// bytes each: with rows of a multiple of 256 bytes (all on the same banks), rows shift
// by 2 * (k & 7) chunks, so the two chunks land on disjoint halves of the 16 groups
// of four banks (k & 7 kept both within the same 8 groups: half of the LDS cycles of
// the 256-wide e4m3 tiles were bank conflicts, counted by SQ_LDS_BANK_CONFLICT; none
// now); rows of 128 bytes shift by k & 7; 192-byte rows alternate between two offsets
// 64 bytes apart, so rows k, k + 2, k + 4, k + 6 shift by (k >> 1) & 3.
template <int RB, int EB>
__device__ __forceinline__ int km_swizzle(int k) {
  if constexpr (EB == 2) {
    if constexpr (RB % 256 == 0) return (k & 3) << 2;
    else return ((k >> 1) & 1) << 2;
  } else {
    if constexpr (RB % 256 == 0) return (k & 7) << 1;
    else if constexpr (RB % 128 == 0) return k & 7;
    else return (k >> 1) & 3;
  }
}
template <int RB, int EB>
__device__ __forceinline__ int km_index(int k, int ch) {
  return k * (RB / 16) + (ch ^ km_swizzle<RB, EB>(k));
}

// One operand tile of R rows (r-major) or R columns (k-major) by SK k per stage of
// EB-byte elements, filled by NW waves (64 chunks of 16 B per instruction). With KEEP
// the lanes' chunk offsets are computed once and held in registers; otherwise they
// are recomputed at every issue from an opaque lane id (a few integer operations per
// instruction), which frees 2 * kN registers for tiles that would otherwise spill.
// EXT: the clip along the operand's memory rows (tile rows r-major, k k-major) is the
// buffer's extent, which leaves one 32-bit compare per chunk for the other axis, and the
// wave index is uniform (LDS destinations in SGPRs); otherwise every chunk compares both
// coordinates. Measured on the 256 x 256 tiles (logits, dW): 1-5% faster; on the dX tiles:
// 2.5% slower at P = 24576, so they keep the per-chunk compares.
template <int R, bool KMAJ, int NW, int SK, int EB, bool KEEP = true, bool EXT = false>
struct DmaTile {
  static constexpr int CPR = SK * EB / 16;  // chunks per r-major row
  static constexpr int RB = R * EB;         // bytes per k-major row
  static constexpr int EPC = 16 / EB;       // elements per chunk
  static_assert((R * SK * EB) % (1024 * NW) == 0 && (CPR == 4 || CPR == 8) &&
                    (!KMAJ || RB % 256 == 0 || RB == 384 || (EB == 1 && (RB % 128 == 0 || RB == 192))),
                "tile shape");
  static_assert(KEEP || EXT, "recomputed offsets come with the extent clip");
  static constexpr int kN = R * SK * EB / (1024 * NW);  // DMA instructions per wave per stage
  int off[KEEP ? kN : 1];  // byte offset of the lane's chunk from the tile origin
  // the chunk's coordinates for the clip: with EXT its k (r-major) or first column
  // (k-major); otherwise (k << 16) | row (r-major) or (row << 16) | first column (k-major)
  int kr[KEEP ? kN : 1];
  int w;    // index of this wave among the NW that fill the tile
  int ldb;  // bytes per operand row in memory (ld * EB)
  int64_t ld;
  // (k, r) of chunk i of this wave for lane `lane`
  __device__ __forceinline__ static void chunk(int wv, int i, int lane, int& k, int& r) {
    const int q = 64 * (wv * kN + i) + lane;  // linear LDS chunk this lane fills
    if constexpr (!KMAJ) {
      r = q / CPR;
      k = ((q % CPR) ^ rm_swizzle<CPR>(r)) * EPC;
    } else {
      k = q / (RB / 16);
      r = ((q % (RB / 16)) ^ km_swizzle<RB, EB>(k)) * EPC;
    }
  }
  __device__ __forceinline__ void init(int64_t ld_, int wave) {
    w = wave;
    ld = ld_;
    ldb = (int)(ld_ * EB);
    if constexpr (KEEP) {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        int k, r;
        chunk(w, i, lane, k, r);
        kr[i] = EXT ? (KMAJ ? r : k) : ((k << 16) | r);
        off[i] = (int)((KMAJ ? (int64_t)k * ld + r : (int64_t)r * ld + k) * EB);
      }
    }
  }
  // base: address of tile element (0, 0) of this stage; rows_valid / k_valid clip the
  // tile (a clipped chunk reads zeros). With EXT, a chunk of a memory row at or past the
  // last valid one starts at or beyond the extent (every chunk lies within its row), and
  // the extent never needs to reach past the tile's SK (k-major) or R (r-major) rows.
  __device__ __forceinline__ void issue(const void* base, int64_t rows_valid, int64_t k_valid,
                                        uint4* tile) const {
    constexpr int kLines = KMAJ ? SK : R, kLim = KMAJ ? R : SK;
    const int64_t lines = KMAJ ? k_valid : rows_valid, cv = KMAJ ? rows_valid : k_valid;
    const int lc = lines <= 0 ? 0 : (lines >= kLines ? kLines : (int)lines);
    const int lim = cv <= 0 ? 0 : (cv >= kLim ? kLim : (int)cv);
    const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                                        EXT ? lc * ldb : kOOB, 0x00020000);
    int lane = 0;
    if constexpr (!KEEP) {
      lane = threadIdx.x & 63;
      asm volatile("" : "+v"(lane));  // keep the recomputation here, not hoisted into registers
    }
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      int o;
      bool in;
      if constexpr (KEEP) {
        o = off[i];
        in = EXT ? kr[i] < lim : ((kr[i] >> 16) < k_valid && (kr[i] & 0xffff) < rows_valid);
      } else {
        int kk, rr;
        chunk(w, i, lane, kk, rr);
        o = (int)(KMAJ ? kk * (int)ld + rr : rr * (int)ld + kk) * EB;
        in = (KMAJ ? rr : kk) < lim;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + (w * kN + i) * 64), 16,
          in ? o : kOOB, 0, 0, 0);
    }
  }
};

// This lane's fragment (k-step ks of the stage) for tile row/column `r_lane` (r_blk:
// first row/column of its 32-block): 8 consecutive bf16 k or 32 consecutive e4m3 k.
template <int R, bool KMAJ, int SK, int EB>
__device__ __forceinline__ typename MfmaElem<EB>::frag_t read_frag(const uint4* tile, int r_lane,
                                                               int r_blk, int ks, int lane) {
  constexpr int CPR = SK * EB / 16, RB = R * EB;
  const char* base = reinterpret_cast<const char*>(tile);
  if constexpr (EB == 2) {
    if constexpr (!KMAJ) {
      return __builtin_bit_cast(bf16x8_t, tile[rm_index<CPR>(r_lane, 2 * ks + (lane >> 5))]);
    } else {
      const int G = lane >> 4, a = lane & 15;
      const int c = r_blk + 16 * (G & 1) + 4 * (a & 3);  // column this lane points at
      i16x4_t h[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int k = 16 * ks + 8 * (G >> 1) + 4 * h2 + (a >> 2);
        const int byte = km_index<RB, EB>(k, c >> 3) * 16 + (c & 7) * 2;
        h[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(base + byte));
      }
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      const i16x8_t v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  } else {
    if constexpr (!KMAJ) {
      const int ch = 4 * ks + 2 * (lane >> 5);
      const uint4 lo = tile[rm_index<CPR>(r_lane, ch)], hi = tile[rm_index<CPR>(r_lane, ch + 1)];
      const i32x8_t v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      return v;
    } else {
      const int G = lane >> 4, a = lane & 15;
      const int c = r_blk + 16 * (G & 1) + 8 * (a & 1);  // 8 columns this lane points at
      i32x2_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = 64 * ks + 32 * (G >> 1) + 8 * q + (a >> 1);
        const int byte = km_index<RB, EB>(k, c >> 4) * 16 + (c & 15);
        h[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(base + byte));
      }
      const i32x8_t v = {h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
      return v;
    }
  }
}

template <int EB>
__device__ __forceinline__ void mfma(const typename MfmaElem<EB>::frag_t& b, const typename MfmaElem<EB>::frag_t& a,
                                     f32x16_t& acc) {
  if constexpr (EB == 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
  else  // formats 0/0: both operands e4m3; E8M0 scales of 127 are 2^0
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc, 0, 0, 0, 127, 0, 127);
}

// Persistent kernel: each workgroup takes the work units (output tile, k-split)
// u = blockIdx.x, blockIdx.x + gridDim.x, ... and streams their k-stages through one
// NS-deep LDS ring without a break between units: the first stages of the next unit
// are already in flight while the current unit finishes and stores its tile.
// BM x BN tile per unit, WGM x WGN waves; OCC workgroups share a CU. The A operand
// has an NS-deep ring, the B operand an NSB-deep one (NSB <= NS): an operand that
// streams from HBM can run further ahead than one that stays in the caches. IL: issue
// the fragment reads one per MFMA (sched_group_barrier) instead of leaving the
// interleave to the compiler; which is faster depends on the product (measured).
// EB: bytes per operand element (2: bf16; 1: e4m3, whose products are multiplied by
// *scale, a device value, before they are stored).
template <int BM, int BN, int WGM, int WGN, bool A_KM, bool B_KM, int OUT, int NS, int OCC,
          int SK, int NSB, bool IL, int EB>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void k_gemm_mfma(
    const void* __restrict__ A, int64_t lda, const void* __restrict__ B, int64_t ldb,
    void* __restrict__ Cout, int64_t ldc, int64_t M, int64_t N, int64_t K, int64_t kps,
    int64_t split_stride, int splits, const float* __restrict__ scale, DwOut dwo) {
  using frag_t = typename MfmaElem<EB>::frag_t;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tiles are whole 32x32 MFMA blocks");
  constexpr int A_SLOT = BM * SK * EB / 16;  // uint4 per A stage
  constexpr int B_SLOT = BN * SK * EB / 16;  // uint4 per B stage
  constexpr int LA = BM * SK * EB / (1024 * NW), LB = BN * SK * EB / (1024 * NW);  // DMA per wave
  constexpr int KS = SK / MfmaElem<EB>::kMfmaK;  // MFMA k-steps per stage
  // Each step issues A then B (equal depths) or B then A (B shallower). Waiting for
  // stage g + 1 leaves in flight what was issued after its later half: whole steps,
  // plus one A group when B runs shallower.
  constexpr int WAIT = NSB < NS ? LA + (NSB - 2) * (LA + LB) : (NS - 2) * (LA + LB);
  constexpr int WAIT0 = (NSB - 1) * LB + (NS - 1) * LA;  // prologue: stage 0 landed
  // KS even: the last k-step of a stage reads fragment buffer 1 while the next stage's
  // first fragments go to buffer 0.
  static_assert(KS >= 2 && KS % 2 == 0 && NSB >= 2 && NSB <= NS && WAIT0 < 64, "pipeline shape");
  // Equal depths: stage s holds its A tile then its B tile (one slot of A_SLOT + B_SLOT);
  // otherwise an A ring followed by a B ring. A bf16 output whose wave slices are 64
  // columns wide goes out through 4 KB of LDS per wave past the ring, when that fits
  // beside it (one workgroup per CU, 160 KB): see store_acc_bf16_lds.
  constexpr int kRing = NS * A_SLOT + NSB * B_SLOT;
  constexpr bool kStaged = OUT == kOutBF16 && TN == 2 && OCC == 1 && (kRing + NW * 256) * 16 <= 160 * 1024;
  __shared__ uint4 lds[kRing + (kStaged ? NW * 256 : 0)];
  auto a_slot = [&](int i) { return lds + (NSB == NS ? i * (A_SLOT + B_SLOT) : i * A_SLOT); };
  auto b_slot = [&](int i) {
    return lds + (NSB == NS ? i * (A_SLOT + B_SLOT) + A_SLOT : NS * A_SLOT + i * B_SLOT);
  };

  // 256 x 256 tiles (logits, dW) clip their ring loads by the buffer extent (see DmaTile)
  constexpr bool kExt = BM == BN;
  const int lane = threadIdx.x & 63;
  const int wid = kExt ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
  const int wm = wid / WGN, wn = wid % WGN;
  const int nbx = (int)((N + BN - 1) / BN), nby = (int)((M + BM - 1) / BM);
  const int ntiles = nbx * nby;
  // kOutDW: dwo.whole whole units, then the other tiles' k-split units
  const int whole = OUT == kOutDW ? dwo.whole : 0;
  const int nunits = whole + (ntiles - whole) * splits;
  const int G = gridDim.x;
  if ((int)blockIdx.x >= nunits) return;
  const int my_units = (nunits - 1 - (int)blockIdx.x) / G + 1;
  const int nk_split = (int)(kps / SK);                  // stages of a split unit
  const int nk_whole = (int)((K + SK - 1) / SK);         // stages of a whole unit

  struct Unit {
    int64_t m0, n0, kb, ke;
    int nk;     // stages
    int split;  // k-range index; -1: a whole unit (kOutDW)
  };
  const int gm = group_rows(nbx, (int64_t)BM * BN * (OUT == kOutBF16 ? 2 : 4));
  auto unit = [&](int i) {
    const int u = (int)blockIdx.x + i * G;
    int tm, tn, sp;
    Unit c;
    if constexpr (OUT == kOutDW) {
      // XCD-contiguous renumbering within each kind; tiles row-major (nbx <= 4)
      int t;
      if (u < whole) {
        t = xcd_order(u, whole);
        sp = -1;
      } else {
        const int rem = ntiles - whole;
        const int lid = xcd_order(u - whole, rem * splits);
        sp = lid / rem;
        t = whole + (lid - sp * rem);
      }
      tm = t / nbx;
      tn = t - tm * nbx;
    } else {
      unit_of(u, nby, nbx, splits, gm, tm, tn, sp);
    }
    c.m0 = (int64_t)tm * BM;
    c.n0 = (int64_t)tn * BN;
    c.split = sp;
    if (sp < 0) {
      c.kb = 0;
      c.ke = K;
      c.nk = nk_whole;
    } else {
      c.kb = (int64_t)sp * kps;
      c.ke = K < c.kb + kps ? K : c.kb + kps;
      c.nk = nk_split;
    }
    return c;
  };

  // e4m3 waves with 8 accumulator blocks recompute their DMA offsets: their fragments
  // are twice bf16's, and spilled registers would be reloaded with vector loads that
  // wait on the DMA queue (measured 1.3x slower dW at S2-late shapes)
  constexpr bool kKeepOffsets = EB == 2 || TM * TN < 8;
  DmaTile<BM, A_KM, NW, SK, EB, kKeepOffsets, kExt> ta;
  DmaTile<BN, B_KM, NW, SK, EB, kKeepOffsets, kExt> tb;
  const char* const Ab = static_cast<const char*>(A);
  const char* const Bb = static_cast<const char*>(B);
  ta.init(lda, wid);
  tb.init(ldb, wid);
  // Issue cursors (unit iu, stage is of that unit), one per operand. Past the last unit,
  // stages are issued fully clipped (zeros, no memory traffic) so every wait count is
  // constant.
  struct Cursor {
    int iu, is;
    Unit c;
  };
  Cursor ca{0, 0, unit(0)};
  Cursor cb = ca;  // B's cursor when NSB < NS
  auto advance = [&](Cursor& q) {
    if (++q.is == q.c.nk) {
      q.is = 0;
      ++q.iu;
      if (q.iu < my_units) q.c = unit(q.iu);
    }
  };
  auto issue_a = [&](int slot_idx) {
    const int64_t k0 = ca.c.kb + (int64_t)ca.is * SK;
    const int64_t kv = ca.iu < my_units ? ca.c.ke - k0 : 0;
    ta.issue(Ab + (A_KM ? k0 * lda + ca.c.m0 : ca.c.m0 * lda + k0) * EB, M - ca.c.m0, kv,
             a_slot(slot_idx));
  };
  auto issue_b = [&](int slot_idx) {
    const int64_t k0 = cb.c.kb + (int64_t)cb.is * SK;
    const int64_t kv = cb.iu < my_units ? cb.c.ke - k0 : 0;
    tb.issue(Bb + (B_KM ? k0 * ldb + cb.c.n0 : cb.c.n0 * ldb + k0) * EB, N - cb.c.n0, kv,
             b_slot(slot_idx));
  };
  // With equal depths both operands of a stage go out together from one cursor, A then
  // B (the wait counts are symmetric then), which keeps the second cursor's registers
  // free.
  auto issue_stage = [&](int slot_idx) {
    const int64_t k0 = ca.c.kb + (int64_t)ca.is * SK;
    const int64_t kv = ca.iu < my_units ? ca.c.ke - k0 : 0;
    ta.issue(Ab + (A_KM ? k0 * lda + ca.c.m0 : ca.c.m0 * lda + k0) * EB, M - ca.c.m0, kv,
             a_slot(slot_idx));
    tb.issue(Bb + (B_KM ? k0 * ldb + ca.c.n0 : ca.c.n0 * ldb + k0) * EB, N - ca.c.n0, kv,
             b_slot(slot_idx));
  };
  // The issue functions leave the cursors where they are; this moves them past what was
  // issued (a unit change is a branch, so it goes after the MFMAs an issue shares a block
  // with).
  auto advance_issued = [&]() {
    advance(ca);
    if constexpr (NSB != NS) advance(cb);
  };

  const int arow = wm * WM;  // wave's first row / column in the tile
  const int bcol = wn * WN;
  const int l32 = lane & 31;
  frag_t fa[2][TM], fb[2][TN];
  auto read_frags = [&](int g, int ks, int buf) {
    const uint4* as = a_slot(g % NS);
    const uint4* bs = b_slot(g % NSB);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[buf][i] = read_frag<BM, A_KM, SK, EB>(as, arow + i * 32 + l32, arow + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[buf][j] = read_frag<BN, B_KM, SK, EB>(bs, bcol + j * 32 + l32, bcol + j * 32, ks, lane);
  };
  f32x16_t acc[TM][TN];
  auto mfma_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        mfma<EB>(fb[buf][j], fa[buf][i], acc[i][j]);
  };
  // ds_read instructions per k-step: bf16 1 (r-major) or 2 (k-major) per fragment, e4m3 2 or 4
  constexpr int kReads = (A_KM ? 2 : 1) * (3 - EB) * TM + (B_KM ? 2 : 1) * (3 - EB) * TN;
  constexpr int kMfma = TM * TN;
  auto interleave = [&]() {
    if constexpr (IL) {
      constexpr int pairs = kReads < kMfma ? kReads : kMfma;
#pragma unroll
      for (int g = 0; g < pairs; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      if (kMfma > pairs) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - pairs, 0);
      if (kReads > pairs) __builtin_amdgcn_sched_group_barrier(0x100, kReads - pairs, 0);
    }
  };
  // Products without pinned reads issue the freed slots' ring loads among the last k-step's
  // MFMAs, one or two after each, so the matrix cores keep working while the loads issue
  // (bf16 dW 3-5% faster than issuing them all before that k-step; the e4m3 fragments are
  // twice as wide, and keeping both stages' fragments live at once there spills).
  constexpr bool kIssueAmongMfma = EB == 2 && !IL;
  constexpr int kDma = LA + LB;  // ring loads per wave per stage
  auto interleave_issue = [&]() {
#pragma unroll
    for (int g = 0; g < kMfma; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      const int n = g < kDma % kMfma ? kDma / kMfma + 1 : kDma / kMfma;
      if (n == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      else if (n == 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      else if (n == 3) __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);
      else if (n >= 4) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
    }
  };

  // Prologue: fill every slot (B then A per stage), wait for global stage 0, fetch its
  // first fragments.
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (NSB == NS) {
      issue_stage(s);
      advance(ca);
    } else {
      if (s < NSB) {
        issue_b(s);
        advance(cb);
      }
      issue_a(s);
      advance(ca);
    }
  }
  vm_wait<WAIT0>();
  lds_barrier();
  read_frags(0, 0, 0);

  int g = 0;  // global stage index of this workgroup
  for (int cu = 0; cu < my_units; ++cu) {
    const Unit cc = unit(cu);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int s = 0; s < cc.nk; ++s, ++g) {
      // e4m3: the k-steps before the stage boundary at raised wave priority (products
      // 0.5-1.5% faster); in bf16 it undoes the dW issue interleave (14% slower)
      if constexpr (EB == 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int q = 0; q + 1 < KS; ++q) {
        // k-step q of stage g, with the reads of its k-step q + 1 in its shadow.
        read_frags(g, q + 1, (q + 1) & 1);
        mfma_step(q & 1);
        interleave();
      }
      if constexpr (EB == 1) __builtin_amdgcn_s_setprio(0);
      // Stage g + 1 becomes visible; the slots of stage g have no readers left (all
      // of their fragment sets are in registers), so they take stages g + NSB (B) and
      // g + NS (A).
      vm_wait<WAIT>();
      lds_barrier();
      auto issue_freed = [&]() {
        if constexpr (NSB == NS) {
          issue_stage(g % NS);
        } else {
          issue_b(g % NSB);
          issue_a(g % NS);
        }
      };
      // Last k-step of stage g, with the first reads of stage g + 1 in its shadow
      // (after the last stage these read a slot that is never used: in bounds, ignored).
      if constexpr (kIssueAmongMfma) {
        read_frags(g + 1, 0, 0);
        issue_freed();
        mfma_step((KS - 1) & 1);
        interleave_issue();
        advance_issued();
      } else {
        issue_freed();
        advance_issued();
        read_frags(g + 1, 0, 0);
        mfma_step((KS - 1) & 1);
        interleave();
      }
    }
    if constexpr (EB == 1) {
      const float sc = *scale;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= sc;
    }
    if constexpr (kStaged) {
      store_acc_bf16_lds<TM, TN>(acc, Cout, ldc, M, N, cc.m0 + arow, cc.n0 + bcol, lane,
                                 lds + kRing + wid * 256);
    } else if constexpr (OUT == kOutDW) {
      if (cc.split < 0)
        store_acc_rows_bf16<TM, TN>(acc, dwo.dW, dwo.ldw, dwo.rowmap, M, N, cc.m0 + arow + l32,
                                    cc.n0 + bcol, lane >> 5);
      else
        store_acc<kOutF32Split, TM, TN>(acc, Cout, ldc, M - dwo.r0, N,
                                        cc.m0 - dwo.r0 + arow + l32, cc.n0 + bcol, lane >> 5,
                                        cc.split * split_stride);
    } else {
      store_acc<OUT, TM, TN>(acc, Cout, ldc, M, N, cc.m0 + arow + l32, cc.n0 + bcol, lane >> 5,
                             OUT == kOutF32Split ? (cc.kb / kps) * split_stride : 0);
    }
  }
  // The ring's last loads (of stages past the last unit: zeros) land before the
  // workgroup's LDS is released.
  vm_wait_all();
}

#define SCE_GEMM_INST(BM, BN, WGM, WGN, AK, BK, OUT, NS, OCC, SK, NSB, IL, EB)                 \
  template __global__ void k_gemm_mfma<BM, BN, WGM, WGN, AK, BK, OUT, NS, OCC, SK, NSB, IL, EB>( \
      const void*, int64_t, const void*, int64_t, void*, int64_t, int64_t, int64_t, int64_t,     \
      int64_t, int64_t, int, const float*, DwOut);
SCE_GEMM_INST(256, 256, 2, 4, false, false, kOutBF16, 2, 1, 64, 2, true, 2)
SCE_GEMM_INST(256, 192, 4, 2, false, false, kOutBF16, 2, 1, 64, 2, true, 2)
SCE_GEMM_INST(256, 192, 4, 2, false, false, kOutF32Split, 2, 1, 64, 2, true, 2)
SCE_GEMM_INST(128, 256, 2, 4, false, false, kOutBF16, 3, 2, 32, 3, true, 2)
SCE_GEMM_INST(128, 256, 2, 4, false, false, kOutF32Split, 3, 2, 32, 3, true, 2)
SCE_GEMM_INST(256, 256, 4, 2, true, true, kOutF32Split, 2, 1, 64, 2, false, 2)
SCE_GEMM_INST(256, 256, 4, 2, true, true, kOutDW, 2, 1, 64, 2, false, 2)
SCE_GEMM_INST(256, 256, 2, 4, false, false, kOutBF16, 2, 1, 128, 2, true, 1)
SCE_GEMM_INST(256, 192, 4, 2, false, true, kOutBF16, 2, 1, 128, 2, false, 1)
SCE_GEMM_INST(256, 192, 4, 2, false, true, kOutF32Split, 2, 1, 128, 2, false, 1)
SCE_GEMM_INST(128, 256, 2, 4, false, true, kOutBF16, 2, 1, 128, 2, true, 1)
SCE_GEMM_INST(128, 256, 2, 4, false, true, kOutF32Split, 2, 1, 128, 2, true, 1)
SCE_GEMM_INST(256, 256, 4, 2, true, true, kOutF32Split, 2, 1, 128, 2, false, 1)
SCE_GEMM_INST(256, 256, 4, 2, true, true, kOutDW, 2, 1, 128, 2, false, 1)
#undef SCE_GEMM_INST

template <int BM, int BN, int WGM, int WGN, bool A_KM, bool B_KM, int OUT, int NS, int OCC,
          int SK, int NSB, bool IL, int EB = 2>
static hipError_t run16(const GemmArgs& a, hipStream_t s) {
  const int splits = a.splits > 0 ? a.splits : 1;
  int64_t kps = (a.K + splits - 1) / splits;
  kps = (kps + SK - 1) / SK * SK;
  if (kps == 0) kps = SK;
  const int64_t gx = (a.N + BN - 1) / BN, gy = (a.M + BM - 1) / BM;
  if (gx == 0 || gy == 0) return hipGetLastError();
  const int64_t whole = OUT == kOutDW ? a.dw.whole : 0;
  if (OUT == kOutDW &&
      (gx > 4 || whole < 0 || whole > gx * gy || whole % gx != 0 || a.dw.r0 != (whole / gx) * BM ||
       (whole > 0 && a.dw.dW == nullptr)))
    return hipErrorInvalidValue;
  const int64_t units = whole + (gx * gy - whole) * splits;
  if (units > 0x7fffffff) return hipErrorInvalidValue;
  // One workgroup per compute unit (a multiple of the 8 XCDs keeps every
  // workgroup's units on one XCD), or one per unit when there are fewer.
  const int slots = cu_count() * OCC;
  const int grid = (int)(units < slots ? units : slots);
  if (EB == 1 && a.scale == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN, A_KM, B_KM, OUT, NS, OCC, SK, NSB, IL, EB>),
                     dim3((unsigned)grid), dim3(64 * WGM * WGN), 0, s, a.A, a.lda, a.B, a.ldb, a.C,
                     a.ldc, a.M, a.N, a.K, kps, a.split_stride, splits, a.scale, a.dw);
  return hipGetLastError();
}

// Tile configurations (measured on MI355X with random bf16 inputs at the workload
// shapes):
//  * logits: 256 x 256 tiles, 8 waves (2 x 4, 128 x 64 each, two per SIMD), one
//    workgroup per CU, two LDS stages of 64 k (both operands are r-major, whose 32-k
//    stages would fetch half cache lines);
//  * dX, N a multiple of 192: 256 x 192 tiles, 8 waves (4 x 2, 64 x 96 each), one
//    workgroup per CU, two stages of 64 k: N = 768 gives 4 column tiles, so M = 16384
//    fills the 256 CUs exactly once. bf16: B is the transposed copy of W_C ([d, P], k
//    contiguous), so both operands are r-major and every fragment is read with
//    ds_read_b128 (against W_C read k-major through transposing LDS reads: 11% faster
//    in the step at T = 16384, P = 10240, 12% at T = 49152, P = 24576; the copy costs
//    7 us at the first). e4m3 reads W_C k-major (ds_read_b64_tr_b8): there the r-major
//    operand measured 2-4% faster alone and no faster in the step once its copy is
//    counted;
//  * dX otherwise: 128 x 256 tiles with two workgroups per CU (their epilogues and
//    barrier stalls interleave), three stages of 32 k, 8 waves of 64 x 64;
//  * dW: 256 x 256 tiles, 8 waves (4 x 2, 64 x 128 each), two stages of 64 k, fragment
//    reads scheduled by the compiler (13-20% faster than the 128 x 256 two-per-CU
//    configuration at P = 10240 ... 50304, T = 16384 ... 49152).
constexpr int kTileM = 128, kTileN = 256, kOcc = 2;
constexpr int kWideM = 256, kWideN = 192;
constexpr int kDwM = 256, kDwN = 256;
static bool dx_wide(int64_t N) { return N % kWideN == 0; }

static int splits_for(int64_t M, int64_t N, int64_t K, int max_splits, bool split_costs_pass,
                      int bm, int bn, int occ) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t slots = (int64_t)cu_count() * occ;
  if (split_costs_pass && tiles < slots) return 1;
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= max_splits; ++s) {
    if (s > 1 && K / s < 1024) break;
    const int64_t units = tiles * s;
    const int64_t rounds = (units + slots - 1) / slots;
    const double eff = (double)units / (double)(rounds * slots);
    if (eff >= 0.85) return s;
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
  }
  return best;
}

// dW (M = P, N = d, K = T: few output tiles, long k): the k-split that minimises an
// estimate of the product's time. Units run in whole rounds of one per CU, each round
// streaming ceil(K / s) k at the configuration's full-round rate over the chip (`flops`:
// about 1.0 PFLOP/s measured for bf16; twice that assumed for e4m3, whose MFMA rate is
// twice bf16's); every split adds an fp32 partial of M x N that is written here and read
// once by the reduction (8 bytes per element at about 5 TB/s).
static int gemm_dw_splits(int64_t M, int64_t N, int64_t K, double flops) {
  const int64_t tiles = ((M + kDwM - 1) / kDwM) * ((N + kDwN - 1) / kDwN);
  const int64_t slots = cu_count();
  const double ns_per_k = 2.0 * kDwM * kDwN * (double)slots / flops * 1.0e9;  // one round
  const double ns_per_partial = 8.0 * (double)M * (double)N / 5.0e3;  // 5e12 B/s
  int best = 1;
  double best_ns = 0.0;
  for (int s = 1; s <= 8; ++s) {
    if (s > 1 && K / s < 1024) break;
    const int64_t rounds = (tiles * s + slots - 1) / slots;
    const double ns = (double)rounds * (double)((K + s - 1) / s) * ns_per_k + s * ns_per_partial;
    if (s == 1 || ns < best_ns) {
      best_ns = ns;
      best = s;
    }
  }
  return best;
}

// The dW schedule (DwPlan). When the tiles outnumber the CUs, whole rounds of tiles run
// unsplit and are stored straight into dW, and only the tiles left over are k-split
// (enough ways to spread them over the CUs, as the estimate above picks): the same
// rounds of MFMA work as splitting every tile, with partials for the leftover rows
// alone. Measured at P = 24576, T = 49152: every tile split 7 ways spent 1.85 ms in dW
// plus 0.11 ms summing 7 partials of 75 MB; 255 whole tiles and 33 split 7 ways
// (partials of 2816 rows) replace both. Otherwise (fewer tiles than CUs, or more than
// four column tiles) every tile is split as before.
static DwPlan gemm_dw_plan(int64_t M, int64_t N, int64_t K, double flops) {
  DwPlan p;
  const int64_t nbx = (N + kDwN - 1) / kDwN, nby = (M + kDwM - 1) / kDwM;
  const int64_t tiles = nbx * nby, slots = cu_count();
  if (nbx > 4 || tiles <= slots || K < 1024) {
    p.splits = gemm_dw_splits(M, N, K, flops);
    return p;
  }
  // whole rounds of tiles, trimmed to whole row blocks
  const int64_t whole = (tiles / slots) * slots / nbx * nbx;
  const int64_t rest_rows = M - (whole / nbx) * kDwM;
  p.whole = (int)whole;
  p.r0 = (whole / nbx) * kDwM;
  p.splits = rest_rows > 0 ? gemm_dw_splits(rest_rows, N, K, flops) : 1;
  return p;
}
DwPlan gemm_bf16_dw_plan(int64_t M, int64_t N, int64_t K) { return gemm_dw_plan(M, N, K, 1.0e15); }
DwPlan gemm_fp8_dw_plan(int64_t M, int64_t N, int64_t K) { return gemm_dw_plan(M, N, K, 2.0e15); }

int gemm_bf16_dx_splits(int64_t M, int64_t N, int64_t K) {
  return dx_wide(N) ? splits_for(M, N, K, 4, true, kWideM, kWideN, 1)
                    : splits_for(M, N, K, 4, true, kTileM, kTileN, kOcc);
}

hipError_t launch_gemm_fp8(Gemm kind, const GemmArgs& a, hipStream_t s) {
  switch (kind) {
    case Gemm::Logits: return run16<256, 256, 2, 4, false, false, kOutBF16, 2, 1, 128, 2, true, 1>(a, s);
    case Gemm::DX:
      if (dx_wide(a.N))
        return a.splits > 1
                   ? run16<kWideM, kWideN, 4, 2, false, true, kOutF32Split, 2, 1, 128, 2, false, 1>(a, s)
                   : run16<kWideM, kWideN, 4, 2, false, true, kOutBF16, 2, 1, 128, 2, false, 1>(a, s);
      return a.splits > 1
                 ? run16<kTileM, kTileN, 2, 4, false, true, kOutF32Split, 2, 1, 128, 2, true, 1>(a, s)
                 : run16<kTileM, kTileN, 2, 4, false, true, kOutBF16, 2, 1, 128, 2, true, 1>(a, s);
    case Gemm::DW:
      return a.dw.whole > 0
                 ? run16<kDwM, kDwN, 4, 2, true, true, kOutDW, 2, 1, 128, 2, false, 1>(a, s)
                 : run16<kDwM, kDwN, 4, 2, true, true, kOutF32Split, 2, 1, 128, 2, false, 1>(a, s);
  }
  return hipErrorInvalidValue;
}

int gemm_fp8_dx_splits(int64_t M, int64_t N, int64_t K) {
  return dx_wide(N) ? splits_for(M, N, K, 4, true, kWideM, kWideN, 1)
                    : splits_for(M, N, K, 4, true, kTileM, kTileN, 1);
}

hipError_t launch_gemm_bf16(Gemm kind, const GemmArgs& a, hipStream_t s) {
  switch (kind) {
    case Gemm::Logits: return run16<256, 256, 2, 4, false, false, kOutBF16, 2, 1, 64, 2, true>(a, s);
    case Gemm::DX:
      if (dx_wide(a.N))
        return a.splits > 1
                   ? run16<kWideM, kWideN, 4, 2, false, false, kOutF32Split, 2, 1, 64, 2, true>(a, s)
                   : run16<kWideM, kWideN, 4, 2, false, false, kOutBF16, 2, 1, 64, 2, true>(a, s);
      return a.splits > 1
                 ? run16<kTileM, kTileN, 2, 4, false, false, kOutF32Split, 3, kOcc, 32, 3, true>(a, s)
                 : run16<kTileM, kTileN, 2, 4, false, false, kOutBF16, 3, kOcc, 32, 3, true>(a, s);
    case Gemm::DW:
      return a.dw.whole > 0
                 ? run16<kDwM, kDwN, 4, 2, true, true, kOutDW, 2, 1, 64, 2, false>(a, s)
                 : run16<kDwM, kDwN, 4, 2, true, true, kOutF32Split, 2, 1, 64, 2, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sce
