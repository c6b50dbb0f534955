// C ABI of libsampledce.so: argument checks, workspace layout and the launch
// sequence of the step. Every launch goes to the caller's stream; nothing here
// allocates, synchronises or copies between host and device.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/sampled_ce.h"
#include "common.h"
#include "kernels.h"

namespace sce {
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t gcd64(int64_t a, int64_t b) {
  while (b != 0) {
    const int64_t r = a % b;
    a = b;
    b = r;
  }
  return a < 0 ? -a : a;
}
int64_t mod64(int64_t a, int64_t m) {
  const int64_t r = a % m;
  return r < 0 ? r + m : r;
}

// Byte offsets of every workspace piece.
struct Plan {
  int64_t Peff = 0, ldz = 0;
  int64_t ldwc = 0;   // row pitch of the gathered W_C (elements)
  int64_t ldt = 0;    // bf16: row pitch of W_C's transpose [d, P_eff] (elements)
  int64_t ldg = 0;    // e4m3 step: row pitch of the e4m3 gradient (bytes)
  int splits = 1;     // k-split of the dW product (fp32 partials reduced by the scatter)
  int dw_whole = 0;   // dW tiles stored whole into dW (rows [0, dw_r0) of the candidate order)
  int64_t dw_r0 = 0;  // first row of the k-split dW tiles (their partials hold rows dw_r0..)
  int dx_splits = 1;  // k-split of the dX product (fp32 partials reduced into dX)
  size_t counters = 0, bits = 0, wpre = 0, cand = 0, tpos = 0, ppos = 0, row_loss = 0;
  size_t wc = 0, wt = 0, z = 0, part = 0, total = 0;
  size_t x8 = 0, g8 = 0, scales = 0;  // e4m3 step
};

// full = false: only what the candidate build needs.
Plan make_plan(int64_t T, int64_t d, int64_t V, int64_t P, int dtype, bool full) {
  Plan p;
  // SCE_E4M3_BF16W: the e4m3 step that encodes the candidate rows of bf16 weights itself
  // (every row at P == 0, into W_C)
  const bool own_codes = dtype == SCE_E4M3_BF16W;
  const bool e4m3 = dtype == SCE_E4M3 || own_codes;
  const size_t es = dtype == SCE_BF16 ? 2 : 4;  // logits element; the e4m3 step's are bf16
  const size_t ws = e4m3 ? 1 : es;              // W_C element
  p.Peff = P == 0 ? V : P;
  // e4m3 step: the gradient's rows share this pitch (a multiple of 16 bytes), and the
  // cross-entropy writes every column below it (zeros past P), so a product's 16-element
  // chunks that straddle K read zeros.
  p.ldz = round_up(p.Peff, e4m3 ? 16 : 8);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.counters = take(kCounterWords * sizeof(int32_t));
  p.bits = take((size_t)((V + 31) / 32) * sizeof(uint32_t));
  p.wpre = take((size_t)((V + 31) / 32) * sizeof(int32_t));
  p.cand = take((size_t)(P > 0 ? P : 1) * sizeof(int32_t));
  p.tpos = take((size_t)(T > 0 ? T : 1) * sizeof(int32_t));
  p.ppos = take((size_t)(T > 0 ? T : 1) * sizeof(int32_t));
  p.row_loss = take((size_t)(T > 0 ? T : 1) * sizeof(float));
  if (full) {
    // W_C rows are padded by 64 elements: with d * es a multiple of 512 bytes (d = 768
    // bf16: 1536 B), the logits product measured 15% slower on unpadded rows.
    p.ldwc = P > 0 ? d + 64 : d;
    p.wc = take(P > 0 || own_codes ? (size_t)p.Peff * p.ldwc * ws : 0);
    if (dtype == SCE_BF16) {
      // The dX product's B operand: W_C transposed (W itself at P = 0), k contiguous,
      // rows a multiple of 16 bytes with zeros past P_eff.
      p.ldt = round_up(p.Peff, 8);
      p.wt = take((size_t)d * p.ldt * ws);
    }
    p.z = take((size_t)T * p.ldz * (e4m3 ? 2 : es));
    if (e4m3) {
      p.ldg = p.ldz;
      p.x8 = take((size_t)T * d);
      p.g8 = take((size_t)T * p.ldg);
      p.scales = take(kNumScales * sizeof(float));
      const DwPlan dw = gemm_fp8_dw_plan(p.Peff, d, T);
      p.splits = dw.splits;
      p.dw_whole = dw.whole;
      p.dw_r0 = dw.r0;
      p.dx_splits = gemm_fp8_dx_splits(T, d, p.Peff);
    } else if (dtype == SCE_BF16) {
      const DwPlan dw = gemm_bf16_dw_plan(p.Peff, d, T);
      p.splits = dw.splits;
      p.dw_whole = dw.whole;
      p.dw_r0 = dw.r0;
      p.dx_splits = gemm_bf16_dx_splits(T, d, p.Peff);
    } else {
      p.splits = gemm_f32_splits(p.Peff, d, T);
      p.dx_splits = gemm_f32_splits(T, d, p.Peff);
    }
    // One region serves both products' partials (dX's are reduced before dW runs).
    const size_t dw_part = (size_t)p.splits * (p.Peff - p.dw_r0) * d;
    const size_t dx_part = p.dx_splits > 1 ? (size_t)p.dx_splits * T * d : 0;
    p.part = take((dw_part > dx_part ? dw_part : dx_part) * sizeof(float));
  }
  p.total = off;
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

sce_status check_sizes(int64_t T, int64_t d, int64_t V, int64_t P, int dtype, bool need_d) {
  if (T < 0 || T > INT32_MAX / 2) return SCE_EINVAL;
  if (V < 1 || V > SCE_MAX_V) return SCE_EINVAL;
  if (P < 0 || P > V) return SCE_EINVAL;
  if (P > 0 && V > SCE_MAX_V_SAMPLED) return SCE_EINVAL;
  if (need_d && (d < 8 || d % 8 != 0 || d > SCE_MAX_D)) return SCE_EINVAL;
  if (need_d && T * d > SCE_MAX_TD) return SCE_EINVAL;
  if (dtype != SCE_F32 && dtype != SCE_BF16 && dtype != SCE_E4M3 && dtype != SCE_E4M3_BF16W)
    return SCE_EINVAL;
  if ((dtype == SCE_E4M3 || dtype == SCE_E4M3_BF16W) && need_d && d % 16 != 0) return SCE_EINVAL;
  return SCE_OK;
}

sce_status hip_status(hipError_t e) { return e == hipSuccess ? SCE_OK : SCE_EHIP; }

// Optional stage timing: when enabled, every call records a HIP event on its
// stream at each stage boundary; sce_profile_collect() sums the elapsed times. The
// events are created by sce_profile_enable (never inside a step call); a call claims
// its slot with one atomic increment.
constexpr int kMaxProfiledCalls = 512;
struct Profile {
  std::atomic<bool> on{false};
  std::atomic<int> calls{0};
  int device = -1;  // the device the events were created on
  hipEvent_t ev[kMaxProfiledCalls][SCE_NUM_STAGES + 1] = {};
} g_prof;

struct StageMarks {
  int call = -1;
  hipStream_t s;
  explicit StageMarks(hipStream_t stream) : s(stream) {
    if (!g_prof.on.load(std::memory_order_acquire)) return;
    const int c = g_prof.calls.fetch_add(1, std::memory_order_relaxed);
    if (c < kMaxProfiledCalls) call = c;
  }
  // Marks the boundary before stage `i` (i == SCE_NUM_STAGES: after the last).
  void mark(int i) {
    if (call >= 0) (void)hipEventRecord(g_prof.ev[call][i], s);
  }
};

// Argument checks shared by both candidate-build entry points.
sce_status check_build_args(const int64_t* targets, int64_t T, int64_t V, int64_t P,
                            int64_t stride, const int32_t* candidates_out,
                            const int32_t* target_pos_out) {
  const sce_status st = check_sizes(T, 8, V, P, SCE_F32, false);
  if (st != SCE_OK || P < 1) return SCE_EINVAL;
  if ((T > 0 && (targets == nullptr || target_pos_out == nullptr)) || candidates_out == nullptr)
    return SCE_EINVAL;
  if (gcd64(mod64(stride, V), V) != 1) return SCE_EINVAL;
  return SCE_OK;
}

// The candidate build's launches, given its scratch: counters, the candidate bitmap and
// per-word prefix counts (ceil(V/32) words each), and prefix positions [T] used when the
// caller passes none.
hipError_t enqueue_build(const int64_t* targets, const int64_t* prefix_targets, int64_t T,
                         int64_t V, int64_t P, int64_t stride, int64_t offset,
                         int32_t* candidates_out, int32_t* vocab_pos_out, int32_t* target_pos_out,
                         int32_t* prefix_pos_out, int64_t* aux_out, int32_t* counters,
                         uint32_t* bits, int32_t* wpre, int32_t* ppos_scratch, hipStream_t hs) {
  int32_t* ppos = prefix_pos_out ? prefix_pos_out : ppos_scratch;
  hipError_t e = launch_candidates(targets, prefix_targets, (int)T, (int)V, (int)P,
                                   (int)mod64(stride, V), (int)mod64(offset, V), counters,
                                   candidates_out, bits, wpre, vocab_pos_out, target_pos_out, ppos,
                                   nullptr, 0, nullptr, 0, nullptr, 0, hs);
  if (e == hipSuccess && aux_out) e = launch_write_aux(counters, aux_out, hs);
  return e;
}

// Layout of the no-allocation build's scratch: the counters, the bitmap and prefix
// counts, then (only when the caller passes no prefix_pos_out) prefix positions [T].
struct NoAllocPlan {
  size_t counters = 0, bits = 0, wpre = 0, ppos = 0, total = 0;
};
NoAllocPlan make_noalloc_plan(int64_t T, int64_t V, bool need_ppos) {
  NoAllocPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.counters = take(kCounterWords * sizeof(int32_t));
  p.bits = take((size_t)((V + 31) / 32) * sizeof(uint32_t));
  p.wpre = take((size_t)((V + 31) / 32) * sizeof(int32_t));
  p.ppos = need_ppos ? take((size_t)(T > 0 ? T : 1) * sizeof(int32_t)) : 0;
  p.total = off;
  return p;
}

}  // namespace
}  // namespace sce

// Scratch of sce_build_candidates_noalloc: one copy per GPU, held until the process
// ends. Host code never passes this name to a kernel or a copy (on the host it stands for
// no device address): the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device by noalloc_scratch().
static __device__ __align__(256) unsigned char scratch[SCE_NOALLOC_SCRATCH_BYTES];

namespace sce {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on its first use
// on that device, with that device current).
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace
}  // namespace sce

using namespace sce;

extern "C" {

int sce_abi_version(void) { return 2; }

const char* sce_status_string(int status) {
  switch (status) {
    case SCE_OK: return "SCE_OK";
    case SCE_EINVAL: return "SCE_EINVAL: invalid argument";
    case SCE_EWORKSPACE: return "SCE_EWORKSPACE: workspace missing or too small";
    case SCE_EHIP: return "SCE_EHIP: HIP launch failed";
    default: return "unknown sce_status";
  }
}

sce_status sce_workspace_size(int64_t T, int64_t d, int64_t V, int64_t P, int dtype,
                              size_t* bytes) {
  if (bytes == nullptr) return SCE_EINVAL;
  const sce_status st = check_sizes(T, d, V, P, dtype, true);
  if (st != SCE_OK) return st;
  *bytes = make_plan(T, d, V, P, dtype, true).total;
  return SCE_OK;
}

sce_status sce_build_candidates(const int64_t* targets, const int64_t* prefix_targets, int64_t T,
                                int64_t V, int64_t P, int64_t stride, int64_t offset,
                                int32_t* candidates_out, int32_t* vocab_pos_out,
                                int32_t* target_pos_out, int32_t* prefix_pos_out,
                                int64_t* aux_out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const sce_status st = check_build_args(targets, T, V, P, stride, candidates_out, target_pos_out);
  if (st != SCE_OK) return st;
  const Plan p = make_plan(T, 8, V, P, SCE_F32, false);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return hip_status(enqueue_build(targets, prefix_targets, T, V, P, stride, offset, candidates_out,
                                  vocab_pos_out, target_pos_out, prefix_pos_out, aux_out,
                                  reinterpret_cast<int32_t*>(ws + p.counters),
                                  reinterpret_cast<uint32_t*>(ws + p.bits),
                                  reinterpret_cast<int32_t*>(ws + p.wpre),
                                  reinterpret_cast<int32_t*>(ws + p.ppos),
                                  static_cast<hipStream_t>(stream)));
}

sce_status sce_build_candidates_noalloc(const int64_t* targets, const int64_t* prefix_targets,
                                        int64_t T, int64_t V, int64_t P, int64_t stride,
                                        int64_t offset, int32_t* candidates_out,
                                        int32_t* vocab_pos_out, int32_t* target_pos_out,
                                        int32_t* prefix_pos_out, int64_t* aux_out, void* stream) {
  const sce_status st = check_build_args(targets, T, V, P, stride, candidates_out, target_pos_out);
  if (st != SCE_OK) return st;
  const NoAllocPlan p = make_noalloc_plan(T, V, prefix_pos_out == nullptr);
  if (p.total > (size_t)SCE_NOALLOC_SCRATCH_BYTES) return SCE_EWORKSPACE;
  void* base = nullptr;
  if (noalloc_scratch(&base) != hipSuccess) return SCE_EHIP;
  char* ws = static_cast<char*>(base);
  return hip_status(enqueue_build(targets, prefix_targets, T, V, P, stride, offset, candidates_out,
                                  vocab_pos_out, target_pos_out, prefix_pos_out, aux_out,
                                  reinterpret_cast<int32_t*>(ws + p.counters),
                                  reinterpret_cast<uint32_t*>(ws + p.bits),
                                  reinterpret_cast<int32_t*>(ws + p.wpre),
                                  reinterpret_cast<int32_t*>(ws + p.ppos),
                                  static_cast<hipStream_t>(stream)));
}

// Everything of the bf16 / fp32 step after its candidate stage: logits, CE, dX, dW, the
// scatter and the loss, on the workspace laid out by `p`.
static hipError_t enqueue_products(const Plan& p, char* ws, const void* x, const void* W,
                                   int64_t T, int64_t d, int64_t P, bool bf16, int32_t* counters,
                                   const int32_t* cand, const int32_t* tpos, const int32_t* ppos,
                                   float* row_loss, float* row_lse_out, float* loss, void* dX,
                                   void* dW, int64_t* aux_out, StageMarks& marks, hipStream_t hs) {
  void* Z = ws + p.z;
  float* part = reinterpret_cast<float*>(ws + p.part);
  const void* WC = P > 0 ? static_cast<const void*>(ws + p.wc) : W;
  // dX's B operand: bf16 reads the transposed copy (r-major), f32 W_C itself (k-major)
  const void* dxB = bf16 ? static_cast<const void*>(ws + p.wt) : WC;
  const int64_t dxldb = bf16 ? p.ldt : p.ldwc;
  hipError_t e = hipSuccess;
  // bf16: dX reads W_C transposed; the gather wrote it when P > 0, W's own is made here
  if (bf16 && T > 0 && P == 0)
    e = launch_transpose(WC, p.ldwc, (int)p.Peff, (int)d, 2, ws + p.wt, p.ldt, hs);
  marks.mark(SCE_STAGE_LOGITS);
  if (e == hipSuccess && T > 0) {
    GemmArgs g{x, d, WC, p.ldwc, Z, p.ldz, T, p.Peff, d, 1, 0};
    e = launch_gemm(Gemm::Logits, bf16, g, hs);
  }
  marks.mark(SCE_STAGE_CE);
  if (e == hipSuccess)
    e = launch_ce_rows(Z, p.ldz, (int)T, (int)p.Peff, bf16, tpos, ppos, counters, row_loss,
                       row_lse_out, hs);
  marks.mark(SCE_STAGE_DX);
  if (e == hipSuccess && T > 0) {
    if (p.dx_splits > 1) {
      GemmArgs g{Z, p.ldz, dxB, dxldb, part, d, T, d, p.Peff, p.dx_splits, T * d};
      e = launch_gemm(Gemm::DX, bf16, g, hs);
    } else {
      GemmArgs g{Z, p.ldz, dxB, dxldb, dX, d, T, d, p.Peff, 1, 0};
      e = launch_gemm(Gemm::DX, bf16, g, hs);
    }
  }
  marks.mark(SCE_STAGE_DX_REDUCE);
  if (e == hipSuccess && T > 0 && p.dx_splits > 1)
    e = launch_scatter_rows(part, p.dx_splits, T * d, nullptr, (int)T, (int)d, bf16, dX, nullptr,
                            hs);
  marks.mark(SCE_STAGE_DW);
  if (e == hipSuccess) {
    GemmArgs g{Z, p.ldz, x, d, part, d, p.Peff, d, T, p.splits, (p.Peff - p.dw_r0) * d};
    g.dw = DwOut{dW, d, P > 0 ? cand : nullptr, p.dw_whole, p.dw_r0};
    e = launch_gemm(Gemm::DW, bf16, g, hs);
  }
  marks.mark(SCE_STAGE_SCATTER);
  if (e == hipSuccess) {
    // The k-split candidate rows of dW, r0.. (the whole tiles' rows were stored by the
    // product; the rows outside C were cleared by the remap launch); the launch's extra
    // block also finishes the loss.
    const LossOut fin{row_loss, (int)T, counters, loss, aux_out};
    const int64_t r0 = p.dw_r0;
    e = launch_scatter_rows(part, p.splits, (p.Peff - r0) * d, P > 0 ? cand + r0 : nullptr,
                            (int)(p.Peff - r0), (int)d, bf16,
                            P > 0 ? dW : static_cast<char*>(dW) + r0 * d * (bf16 ? 2 : 4), &fin,
                            hs);
  }
  marks.mark(SCE_NUM_STAGES);
  return e;
}

// Host checks shared by the bf16 / fp32 step entry points.
static sce_status check_step(const void* x, const void* W, const void* labels, int64_t T,
                             int64_t d, int64_t V, int64_t P, int dtype, const float* loss,
                             const void* dX, const void* dW) {
  if (dtype == SCE_E4M3 || dtype == SCE_E4M3_BF16W) return SCE_EINVAL;  // the e4m3 entry points
  const sce_status st = check_sizes(T, d, V, P, dtype, true);
  if (st != SCE_OK) return st;
  if (W == nullptr || loss == nullptr || dW == nullptr) return SCE_EINVAL;
  if (T > 0 && (x == nullptr || labels == nullptr || dX == nullptr)) return SCE_EINVAL;
  if ((x && !aligned16(x)) || !aligned16(W) || (dX && !aligned16(dX)) || !aligned16(dW))
    return SCE_EINVAL;
  return SCE_OK;
}

sce_status sampled_ce_forward_backward(const void* x, const void* W, const int64_t* targets,
                                       const int64_t* prefix_targets, int64_t T, int64_t d,
                                       int64_t V, int64_t P, int64_t stride, int64_t offset,
                                       int dtype, float* loss, void* dX, void* dW,
                                       int32_t* candidates_out, int32_t* target_pos_out,
                                       int32_t* prefix_pos_out, float* row_lse_out,
                                       float* row_loss_out, int64_t* aux_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  sce_status st = check_step(x, W, targets, T, d, V, P, dtype, loss, dX, dW);
  if (st != SCE_OK) return st;
  int64_t s = 1;
  if (P > 0) {
    s = mod64(stride, V);
    if (gcd64(s, V) != 1) return SCE_EINVAL;
  }
  const Plan p = make_plan(T, d, V, P, dtype, true);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;

  const bool bf16 = dtype == SCE_BF16;
  const size_t es = bf16 ? 2 : 4;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + p.bits);
  int32_t* wpre = reinterpret_cast<int32_t*>(ws + p.wpre);
  int32_t* cand = candidates_out ? candidates_out : reinterpret_cast<int32_t*>(ws + p.cand);
  int32_t* tpos = target_pos_out ? target_pos_out : reinterpret_cast<int32_t*>(ws + p.tpos);
  int32_t* ppos = prefix_pos_out ? prefix_pos_out : reinterpret_cast<int32_t*>(ws + p.ppos);
  float* row_loss = row_loss_out ? row_loss_out : reinterpret_cast<float*>(ws + p.row_loss);

  StageMarks marks(hs);
  marks.mark(SCE_STAGE_CANDIDATES);
  hipError_t e = launch_candidates(targets, prefix_targets, (int)T, (int)V, (int)P, (int)s,
                                   (int)mod64(offset, V), counters, cand, bits, wpre, nullptr,
                                   tpos, ppos,
                                   W, (int)(d * es), ws + p.wc, (int)(p.ldwc * es), dW,
                                   (int)(d * es), hs, nullptr, -1, nullptr,
                                   bf16 && T > 0 ? ws + p.wt : nullptr, p.ldt);
  if (e == hipSuccess)
    e = enqueue_products(p, ws, x, W, T, d, P, bf16, counters, cand, tpos, ppos, row_loss,
                         row_lse_out, loss, dX, dW, aux_out, marks, hs);
  return hip_status(e);
}

sce_status sampled_ce_forward_backward_prebuilt(const void* x, const void* W,
                                                const int32_t* candidates,
                                                const int32_t* target_pos,
                                                const int32_t* prefix_pos,
                                                const int64_t* build_aux, int64_t T, int64_t d,
                                                int64_t V, int64_t P, int dtype, float* loss,
                                                void* dX, void* dW, float* row_lse_out,
                                                float* row_loss_out, int64_t* aux_out,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
  sce_status st = check_step(x, W, target_pos, T, d, V, P, dtype, loss, dX, dW);
  if (st != SCE_OK) return st;
  if (P < 1 || candidates == nullptr) return SCE_EINVAL;  // a sampled candidate set only
  const Plan p = make_plan(T, d, V, P, dtype, true);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;

  const bool bf16 = dtype == SCE_BF16;
  const size_t es = bf16 ? 2 : 4;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + p.bits);
  int32_t* cand = reinterpret_cast<int32_t*>(ws + p.cand);
  int32_t* tpos = reinterpret_cast<int32_t*>(ws + p.tpos);
  int32_t* ppos = reinterpret_cast<int32_t*>(ws + p.ppos);
  float* row_loss = row_loss_out ? row_loss_out : reinterpret_cast<float*>(ws + p.row_loss);

  StageMarks marks(hs);
  marks.mark(SCE_STAGE_CANDIDATES);
  hipError_t e = launch_candidates_prebuilt(candidates, target_pos, prefix_pos, build_aux, (int)T,
                                            (int)V, (int)P, counters, cand, bits, tpos, ppos, W,
                                            (int)(d * es), ws + p.wc, (int)(p.ldwc * es), dW,
                                            (int)(d * es), bf16 && T > 0 ? ws + p.wt : nullptr,
                                            p.ldt, hs);
  if (e == hipSuccess)
    e = enqueue_products(p, ws, x, W, T, d, P, bf16, counters, cand, tpos, ppos, row_loss,
                         row_lse_out, loss, dX, dW, aux_out, marks, hs);
  return hip_status(e);
}

// The e4m3 step after its candidate stage: x's quantisation (from the max|x| partials
// the candidate launch left), the three e4m3 products, the CE writing the e4m3 gradient,
// the reductions and the loss. n_max = 2 with prefix targets, else 1.
static hipError_t enqueue_products_fp8(const Plan& p, char* ws, const void* x, const void* W8,
                                       float w_scale, const float* w_scale_dev, int64_t T,
                                       int64_t d, int64_t P, int n_max, int32_t* counters,
                                       int32_t* cand, int32_t* tpos, int32_t* ppos,
                                       float* row_loss, float* row_lse_out, float* loss, void* dX,
                                       void* dW, int64_t* aux_out, float* scales_out,
                                       int amax_parts, StageMarks& marks, hipStream_t hs) {
  float* scales = reinterpret_cast<float*>(ws + p.scales);
  void* Z = ws + p.z;
  uint8_t* x8 = reinterpret_cast<uint8_t*>(ws + p.x8);
  uint8_t* g8 = reinterpret_cast<uint8_t*>(ws + p.g8);
  float* part = reinterpret_cast<float*>(ws + p.part);
  const void* WC = P > 0 ? static_cast<const void*>(ws + p.wc) : W8;

  hipError_t e = launch_quant_x(x, T * d, counters, w_scale, w_scale_dev, x8, scales, scales_out,
                                hs, amax_parts);
  marks.mark(SCE_STAGE_LOGITS);
  if (e == hipSuccess && T > 0) {
    GemmArgs g{x8, d, WC, p.ldwc, Z, p.ldz, T, p.Peff, d, 1, 0, scales + kScaleLogits};
    e = launch_gemm_fp8(Gemm::Logits, g, hs);
  }
  marks.mark(SCE_STAGE_CE);
  if (e == hipSuccess) {
    const G8Out go{g8, p.ldg, n_max, scales, scales_out};
    e = launch_ce_rows_g8(Z, p.ldz, (int)T, (int)p.Peff, tpos, ppos, counters, row_loss,
                          row_lse_out, go, hs);
  }
  marks.mark(SCE_STAGE_DX);
  if (e == hipSuccess && T > 0) {
    if (p.dx_splits > 1) {
      GemmArgs g{g8, p.ldg, WC, p.ldwc, part, d, T, d, p.Peff, p.dx_splits, T * d, scales + kScaleDx};
      e = launch_gemm_fp8(Gemm::DX, g, hs);
    } else {
      GemmArgs g{g8, p.ldg, WC, p.ldwc, dX, d, T, d, p.Peff, 1, 0, scales + kScaleDx};
      e = launch_gemm_fp8(Gemm::DX, g, hs);
    }
  }
  marks.mark(SCE_STAGE_DX_REDUCE);
  if (e == hipSuccess && T > 0 && p.dx_splits > 1)
    e = launch_scatter_rows(part, p.dx_splits, T * d, nullptr, (int)T, (int)d, true, dX, nullptr,
                            hs);
  marks.mark(SCE_STAGE_DW);
  if (e == hipSuccess && T > 0) {
    GemmArgs g{g8, p.ldg, x8, d, part, d, p.Peff, d, T, p.splits, (p.Peff - p.dw_r0) * d,
               scales + kScaleDw};
    g.dw = DwOut{dW, d, P > 0 ? cand : nullptr, p.dw_whole, p.dw_r0};
    e = launch_gemm_fp8(Gemm::DW, g, hs);
  }
  marks.mark(SCE_STAGE_SCATTER);
  if (e == hipSuccess) {
    const LossOut fin{row_loss, (int)T, counters, loss, aux_out};
    // T = 0: no product ran; every candidate row is written as zeros (a sum over no
    // partials), the others were cleared by the remap launch. Otherwise the k-split rows
    // r0.. (the product stored the whole tiles' rows).
    const int64_t r0 = T > 0 ? p.dw_r0 : 0;
    e = launch_scatter_rows(part, T > 0 ? p.splits : 0, (p.Peff - r0) * d,
                            P > 0 ? cand + r0 : nullptr, (int)(p.Peff - r0), (int)d, true,
                            P > 0 ? dW : static_cast<char*>(dW) + r0 * d * 2, &fin, hs);
  }
  marks.mark(SCE_NUM_STAGES);
  return e;
}

// Host checks shared by the e4m3 entry points.
static sce_status check_fp8(const void* x, const void* W8, float w_scale,
                            const float* w_scale_dev, const void* labels, int64_t T, int64_t d,
                            int64_t V, int64_t P, const float* loss, const void* dX,
                            const void* dW) {
  const sce_status st = check_sizes(T, d, V, P, SCE_E4M3, true);
  if (st != SCE_OK) return st;
  if (w_scale_dev == nullptr && (!(w_scale > 0.f) || w_scale > 3.0e38f))
    return SCE_EINVAL;  // also rejects NaN; a device scale is checked on the device
  if (w_scale_dev != nullptr && (reinterpret_cast<uintptr_t>(w_scale_dev) & 3) != 0)
    return SCE_EINVAL;
  if (W8 == nullptr || loss == nullptr || dW == nullptr) return SCE_EINVAL;
  if (T > 0 && (x == nullptr || labels == nullptr || dX == nullptr)) return SCE_EINVAL;
  if ((x && !aligned16(x)) || !aligned16(W8) || (dX && !aligned16(dX)) || !aligned16(dW))
    return SCE_EINVAL;
  return SCE_OK;
}

sce_status sampled_ce_forward_backward_fp8(const void* x, const void* W8, float w_scale,
                                           const float* w_scale_dev,
                                           const int64_t* targets, const int64_t* prefix_targets,
                                           int64_t T, int64_t d, int64_t V, int64_t P,
                                           int64_t stride, int64_t offset, float* loss, void* dX,
                                           void* dW, int32_t* candidates_out,
                                           int32_t* target_pos_out, int32_t* prefix_pos_out,
                                           float* row_lse_out, float* row_loss_out,
                                           int64_t* aux_out, float* scales_out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  sce_status st = check_fp8(x, W8, w_scale, w_scale_dev, targets, T, d, V, P, loss, dX, dW);
  if (st != SCE_OK) return st;
  int64_t s = 1;
  if (P > 0) {
    s = mod64(stride, V);
    if (gcd64(s, V) != 1) return SCE_EINVAL;
  }
  const Plan p = make_plan(T, d, V, P, SCE_E4M3, true);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;

  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + p.bits);
  int32_t* wpre = reinterpret_cast<int32_t*>(ws + p.wpre);
  int32_t* cand = candidates_out ? candidates_out : reinterpret_cast<int32_t*>(ws + p.cand);
  int32_t* tpos = target_pos_out ? target_pos_out : reinterpret_cast<int32_t*>(ws + p.tpos);
  int32_t* ppos = prefix_pos_out ? prefix_pos_out : reinterpret_cast<int32_t*>(ws + p.ppos);
  float* row_loss = row_loss_out ? row_loss_out : reinterpret_cast<float*>(ws + p.row_loss);

  StageMarks marks(hs);
  marks.mark(SCE_STAGE_CANDIDATES);
  int amax_parts = 0;  // max|x| partials, taken beside the candidate build
  hipError_t e = launch_candidates(targets, prefix_targets, (int)T, (int)V, (int)P, (int)s,
                                   (int)mod64(offset, V), counters, cand, bits, wpre, nullptr,
                                   tpos, ppos,
                                   W8, (int)d, ws + p.wc, (int)p.ldwc, dW, (int)(d * 2), hs,
                                   x, T * d, &amax_parts);
  if (e == hipSuccess)
    e = enqueue_products_fp8(p, ws, x, W8, w_scale, w_scale_dev, T, d, P,
                             prefix_targets ? 2 : 1, counters, cand, tpos, ppos, row_loss,
                             row_lse_out, loss, dX, dW, aux_out, scales_out, amax_parts, marks,
                             hs);
  return hip_status(e);
}

sce_status sampled_ce_forward_backward_fp8_bf16w(
    const void* x, const void* W, const int64_t* targets, const int64_t* prefix_targets, int64_t T,
    int64_t d, int64_t V, int64_t P, int64_t stride, int64_t offset, float* loss, void* dX,
    void* dW, int32_t* candidates_out, int32_t* target_pos_out, int32_t* prefix_pos_out,
    float* row_lse_out, float* row_loss_out, int64_t* aux_out, float* scales_out, void* workspace,
    size_t workspace_bytes, void* stream) {
  sce_status st = check_fp8(x, W, 1.f, nullptr, targets, T, d, V, P, loss, dX, dW);
  if (st != SCE_OK) return st;
  int64_t s = 1;
  if (P > 0) {
    s = mod64(stride, V);
    if (gcd64(s, V) != 1) return SCE_EINVAL;
  }
  const Plan p = make_plan(T, d, V, P, SCE_E4M3_BF16W, true);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;

  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + p.bits);
  int32_t* wpre = reinterpret_cast<int32_t*>(ws + p.wpre);
  int32_t* cand = candidates_out ? candidates_out : reinterpret_cast<int32_t*>(ws + p.cand);
  int32_t* tpos = target_pos_out ? target_pos_out : reinterpret_cast<int32_t*>(ws + p.tpos);
  int32_t* ppos = prefix_pos_out ? prefix_pos_out : reinterpret_cast<int32_t*>(ws + p.ppos);
  float* row_loss = row_loss_out ? row_loss_out : reinterpret_cast<float*>(ws + p.row_loss);
  float* scales = reinterpret_cast<float*>(ws + p.scales);

  StageMarks marks(hs);
  marks.mark(SCE_STAGE_CANDIDATES);
  int amax_parts = 0;  // max|x| partials, and max|W| partials, taken beside the build
  CacheEncode enc;
  enc.scale_slot = scales + kScaleWCache;
  enc.scale_out = scales_out ? scales_out + 2 : nullptr;
  hipError_t e = launch_candidates(targets, prefix_targets, (int)T, (int)V, (int)P, (int)s,
                                   (int)mod64(offset, V), counters, cand, bits, wpre, nullptr,
                                   tpos, ppos, W, (int)(d * 2), ws + p.wc, (int)p.ldwc, dW,
                                   (int)(d * 2), hs, x, T * d, &amax_parts, nullptr, 0, &enc);
  // the products read the codes the gather wrote (every row at P == 0), with s_w as the
  // cache's scale, read on the device
  if (e == hipSuccess)
    e = enqueue_products_fp8(p, ws, x, ws + p.wc, 1.f, scales + kScaleWCache, T, d, P,
                             prefix_targets ? 2 : 1, counters, cand, tpos, ppos, row_loss,
                             row_lse_out, loss, dX, dW, aux_out, scales_out, amax_parts, marks,
                             hs);
  return hip_status(e);
}

sce_status sampled_ce_forward_backward_fp8_prebuilt(
    const void* x, const void* W8, float w_scale, const float* w_scale_dev,
    const int32_t* candidates, const int32_t* target_pos, const int32_t* prefix_pos,
    const int64_t* build_aux, int64_t T, int64_t d, int64_t V, int64_t P, float* loss, void* dX,
    void* dW, float* row_lse_out, float* row_loss_out, int64_t* aux_out, float* scales_out,
    void* workspace, size_t workspace_bytes, void* stream) {
  sce_status st = check_fp8(x, W8, w_scale, w_scale_dev, target_pos, T, d, V, P, loss, dX, dW);
  if (st != SCE_OK) return st;
  if (P < 1 || candidates == nullptr) return SCE_EINVAL;  // a sampled candidate set only
  const Plan p = make_plan(T, d, V, P, SCE_E4M3, true);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;

  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + p.bits);
  int32_t* cand = reinterpret_cast<int32_t*>(ws + p.cand);
  int32_t* tpos = reinterpret_cast<int32_t*>(ws + p.tpos);
  int32_t* ppos = reinterpret_cast<int32_t*>(ws + p.ppos);
  float* row_loss = row_loss_out ? row_loss_out : reinterpret_cast<float*>(ws + p.row_loss);

  StageMarks marks(hs);
  marks.mark(SCE_STAGE_CANDIDATES);
  int amax_parts = 0;
  hipError_t e = launch_candidates_prebuilt(candidates, target_pos, prefix_pos, build_aux, (int)T,
                                            (int)V, (int)P, counters, cand, bits, tpos, ppos, W8,
                                            (int)d, ws + p.wc, (int)p.ldwc, dW, (int)(d * 2),
                                            nullptr, 0, hs, x, T * d, &amax_parts);
  if (e == hipSuccess)
    e = enqueue_products_fp8(p, ws, x, W8, w_scale, w_scale_dev, T, d, P, prefix_pos ? 2 : 1,
                             counters, cand, tpos, ppos, row_loss, row_lse_out, loss, dX, dW,
                             aux_out, scales_out, amax_parts, marks, hs);
  return hip_status(e);
}

sce_status sce_refresh_e4m3_cache(const void* W, int64_t V, int64_t d, void* W8_out,
                                  float* w_scale_out, int32_t* status_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  static_assert((kAmaxX + kAmaxSlots) * sizeof(int32_t) <= SCE_REFRESH_WORKSPACE_BYTES,
                "the refresh's partial maxima fit its workspace");
  if (V < 1 || V > SCE_MAX_V || d < 16 || d > SCE_MAX_D || d % 16 != 0) return SCE_EINVAL;
  if (W == nullptr || W8_out == nullptr || w_scale_out == nullptr) return SCE_EINVAL;
  if (!aligned16(W) || !aligned16(W8_out) || (reinterpret_cast<uintptr_t>(w_scale_out) & 3) ||
      (reinterpret_cast<uintptr_t>(status_out) & 3))
    return SCE_EINVAL;
  if (workspace == nullptr || workspace_bytes < SCE_REFRESH_WORKSPACE_BYTES ||
      (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return SCE_EWORKSPACE;
  return hip_status(launch_refresh_e4m3(W, V * d, W8_out, w_scale_out, status_out,
                                        static_cast<int32_t*>(workspace),
                                        static_cast<hipStream_t>(stream)));
}

// ---- building blocks on their own ---------------------------------------------

namespace {
struct CePlan {
  size_t counters = 0, tpos = 0, ppos = 0, row_loss = 0, total = 0;
};
CePlan make_ce_plan(int64_t T) {
  CePlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t n = (size_t)(T > 0 ? T : 1);
  p.counters = take(kCounterWords * sizeof(int32_t));
  p.tpos = take(n * sizeof(int32_t));
  p.ppos = take(n * sizeof(int32_t));
  p.row_loss = take(n * sizeof(float));
  p.total = off;
  return p;
}
}  // namespace

sce_status sce_ce_rows_workspace_size(int64_t T, size_t* bytes) {
  if (bytes == nullptr || T < 0 || T > INT32_MAX / 2) return SCE_EINVAL;
  *bytes = make_ce_plan(T).total;
  return SCE_OK;
}

sce_status sce_ce_rows(void* Z, int64_t ldz, int64_t T, int64_t P, int dtype,
                       const int32_t* target_pos, const int32_t* prefix_pos, float* loss,
                       float* row_loss_out, float* row_lse_out, int64_t* aux_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (T < 0 || T > INT32_MAX / 2 || P < 1 || P > SCE_MAX_V) return SCE_EINVAL;
  if (ldz < P || ldz % 8 != 0 || ldz > (int64_t)SCE_MAX_V + 8) return SCE_EINVAL;
  if (dtype != SCE_F32 && dtype != SCE_BF16) return SCE_EINVAL;
  if (loss == nullptr || (T > 0 && (Z == nullptr || target_pos == nullptr))) return SCE_EINVAL;
  if (Z && !aligned16(Z)) return SCE_EINVAL;
  const CePlan p = make_ce_plan(T);
  if (workspace == nullptr || workspace_bytes < p.total) return SCE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SCE_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  int32_t* tpos = reinterpret_cast<int32_t*>(ws + p.tpos);
  int32_t* ppos = reinterpret_cast<int32_t*>(ws + p.ppos);
  float* row_loss = row_loss_out ? row_loss_out : reinterpret_cast<float*>(ws + p.row_loss);
  const bool bf16 = dtype == SCE_BF16;
  hipError_t e = launch_ce_prep(target_pos, prefix_pos, (int)T, (int)P, tpos, ppos, counters, hs);
  if (e == hipSuccess)
    e = launch_ce_rows(Z, ldz, (int)T, (int)P, bf16, tpos, ppos, counters, row_loss, row_lse_out,
                       hs);
  if (e == hipSuccess) {
    // the scatter launch with no rows: only its loss block runs
    const LossOut fin{row_loss, (int)T, counters, loss, aux_out};
    e = launch_scatter_rows(nullptr, 0, 0, nullptr, 0, 8, bf16, nullptr, &fin, hs);
  }
  return hip_status(e);
}

sce_status sce_gather_rows(const void* W, int64_t V, int64_t d, const int32_t* idx, int64_t n,
                           int dtype, void* out, int64_t ld_out, int32_t* status_out,
                           void* stream) {
  if (V < 1 || n < 0 || n > INT32_MAX / 2 || d < 8 || d % 8 != 0 || d > SCE_MAX_D) return SCE_EINVAL;
  if (dtype != SCE_F32 && dtype != SCE_BF16) return SCE_EINVAL;
  if (ld_out < d || ld_out % 8 != 0) return SCE_EINVAL;
  if (n > 0 && (W == nullptr || idx == nullptr || out == nullptr)) return SCE_EINVAL;
  if ((W && !aligned16(W)) || (out && !aligned16(out))) return SCE_EINVAL;
  if (n == 0) return SCE_OK;
  const int64_t es = dtype == SCE_BF16 ? 2 : 4;
  return hip_status(launch_gather_checked(W, V, idx, (int)n, (int)(d * es), out, ld_out * es,
                                          status_out, static_cast<hipStream_t>(stream)));
}

sce_status sce_profile_enable(int on) {
  if (on && !g_prof.on.load()) {
    // a new timing window; the events are made once, on the current device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SCE_EHIP;
    if (g_prof.device != dev) {
      for (int c = 0; c < kMaxProfiledCalls; ++c)
        for (int i = 0; i <= SCE_NUM_STAGES; ++i) {
          if (g_prof.device >= 0) (void)hipEventDestroy(g_prof.ev[c][i]);
          if (hipEventCreate(&g_prof.ev[c][i]) != hipSuccess) {
            g_prof.device = -1;
            return SCE_EHIP;
          }
        }
      g_prof.device = dev;
    }
    g_prof.calls.store(0);
  }
  g_prof.on.store(on != 0, std::memory_order_release);  // disabling keeps the record
  return SCE_OK;
}

sce_status sce_profile_collect(double* stage_ms, int nstages, int* ncalls) {
  if (stage_ms == nullptr || nstages < SCE_NUM_STAGES) return SCE_EINVAL;
  for (int i = 0; i < nstages; ++i) stage_ms[i] = 0.0;
  int n = g_prof.calls.load();
  if (n > kMaxProfiledCalls) n = kMaxProfiledCalls;
  for (int c = 0; c < n; ++c) {
    if (hipEventSynchronize(g_prof.ev[c][SCE_NUM_STAGES]) != hipSuccess) return SCE_EHIP;
    for (int i = 0; i < SCE_NUM_STAGES; ++i) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_prof.ev[c][i], g_prof.ev[c][i + 1]) != hipSuccess)
        return SCE_EHIP;
      stage_ms[i] += ms;
    }
  }
  if (ncalls) *ncalls = n;
  g_prof.calls.store(0);
  return SCE_OK;
}

}  // extern "C"
