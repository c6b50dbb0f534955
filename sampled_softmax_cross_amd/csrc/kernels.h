// Launchers shared between the kernel translation units and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sce {

constexpr int kBuildThreads = 1024;

// Byte map of candidate marks: one byte per class, rounded up to 32 classes.
inline int bytemap_bytes(int V) { return (V + 31) / 32 * 32; }

hipError_t launch_candidates(const int64_t* targets, const int64_t* prefix, int T, int V, int P,
                             int stride, int off, uint8_t* bytemap, int32_t* counters,
                             int32_t* C, int32_t* vocab_pos, int32_t* target_pos,
                             int32_t* prefix_pos, hipStream_t s);
hipError_t launch_write_aux(const int32_t* counters, int64_t* aux, hipStream_t s);

// W_C[i, :] = W[C[i], :] (rows of row_bytes, a multiple of 16).
hipError_t launch_gather_rows(const void* W, const int32_t* C, int P, int row_bytes, void* WC,
                              hipStream_t s);
// dW[v, :] = sum over splits of part[s, pos(v), :] (fp32) in dtype, or 0 when pos(v) < 0;
// pos = vocab_pos, or the identity when vocab_pos is null.
hipError_t launch_scatter_rows(const float* part, int splits, int64_t split_stride,
                               const int32_t* vocab_pos, int V, int d, bool bf16, void* dW,
                               hipStream_t s);

// Row-wise cross-entropy forward/backward over Z [T, ldz] (P valid columns), in place.
hipError_t launch_ce_rows(void* Z, int64_t ldz, int T, int P, bool bf16,
                          const int32_t* target_pos, const int32_t* prefix_pos,
                          const int32_t* counters, float* row_loss, float* row_lse,
                          hipStream_t s);
// loss = sum(row_loss) / N (0 when N == 0); optional aux copy.
hipError_t launch_finalize(const float* row_loss, int T, const int32_t* counters, float* loss,
                           int64_t* aux, hipStream_t s);

// GEMMs. Matrices row-major; see gemm.hip for the operand conventions.
enum class Gemm { Logits, DX, DW };
struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int64_t M, N, K;
  int splits;            // split-K factor (DW only)
  int64_t split_stride;  // elements between split slabs of C (DW only)
};
// k-split factor for a GEMM of this shape (1 = no split). bf16 products only; the
// fp32 products use gemm_dw_splits for dW and never split dX.
int gemm_bf16_splits(int64_t M, int64_t N, int64_t K, int max_splits);
int gemm_dw_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(Gemm kind, bool bf16, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16(Gemm kind, const GemmArgs& a, hipStream_t s);

}  // namespace sce
