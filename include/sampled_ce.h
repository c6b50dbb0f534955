/*
 * sampled_ce.h -- C ABI of libsampledce.so: the sampled-softmax cross-entropy
 * LM-head step (forward and backward) on AMD Instinct MI355X (gfx950).
 *
 * The method ("sampled_softmax.py", modded-nanogpt track_1_short, module
 * docstring): the T tokens of one microbatch (hidden states x [T, d]) all share
 * one set C of P output classes, and the training cross-entropy normalises over
 * C rather than over the whole vocabulary of V classes. C is the union of the
 * distinct labels of the microbatch with filler classes ("negatives") read off a
 * fixed cyclic order of the vocabulary, c_k = k * stride mod V (a permutation
 * because gcd(stride, V) = 1), starting at a caller-chosen index. The kernels see
 * C as a P-class vocabulary: logits x @ W[C]^T, labels given as indexes into C.
 * A prefix label whose class did not make it into C gets index -1 and is skipped;
 * such labels never add classes to C. The LM-head gradient covers all V rows and
 * is zero on every row outside C. P = 0 selects the ordinary softmax over all V
 * classes.
 *
 * Conventions shared by every entry point:
 *   - Every array pointer is a DEVICE pointer unless its comment says "host".
 *     The caller owns every buffer; the library never allocates or frees memory.
 *   - Matrices are row-major and densely packed (row stride = row length).
 *   - `dtype` is SCE_BF16 (bfloat16 storage, fp32 accumulation) or SCE_F32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting for it. Nothing is synchronised and no
 *     host<->device copy is made inside a call.
 *   - Errors the host can see are returned synchronously and nothing is enqueued.
 *     Errors only the device can see (a label out of range, more distinct targets
 *     than P) are OR-ed into aux_out[3] (SCE_DEV_* bits); the other outputs of
 *     such a call are unspecified but every access stays in bounds.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Calls that share a workspace must not overlap in time (use one workspace per
 *     stream). Calls with distinct workspaces and outputs are independent.
 */
#ifndef SAMPLED_CE_H
#define SAMPLED_CE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SCE_API __attribute__((visibility("default")))
#else
#define SCE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sce_status {
  SCE_OK = 0,
  SCE_EINVAL = 1,     /* an argument is out of range or a required pointer is NULL */
  SCE_EWORKSPACE = 2, /* workspace NULL or smaller than sce_workspace_size() */
  SCE_EHIP = 3        /* a HIP launch failed (see hipGetLastError) */
} sce_status;

/* In sce_workspace_size: SCE_E4M3 names the fp8 steps that read an e4m3 cache
 * (sampled_ce_forward_backward_fp8 and _fp8_prebuilt), SCE_E4M3_BF16W the fp8 step that
 * encodes the candidate rows of bf16 weights itself (sampled_ce_forward_backward_fp8_bf16w). */
typedef enum sce_dtype { SCE_F32 = 0, SCE_BF16 = 1, SCE_E4M3 = 2, SCE_E4M3_BF16W = 3 } sce_dtype;

/* Device-detected conditions (bits of aux_out[3]). */
#define SCE_DEV_TOO_MANY_TARGETS 1 /* distinct targets > P (the page asserts this never happens) */
#define SCE_DEV_LABEL_RANGE 2      /* a target or prefix target outside [-1, V) */
#define SCE_DEV_SCALE_RANGE 4      /* fp8 step: x not finite, or 0 < max|x| < 2^-100 */

/* Limits checked on the host. */
#define SCE_MAX_V_SAMPLED 131072 /* V limit when P > 0 (two candidate bitmaps held in LDS) */
#define SCE_MAX_V 1048576        /* V limit for the full softmax (32-bit tile offsets) */
#define SCE_MAX_D 16384
#define SCE_MAX_TD (1LL << 34)   /* T * d limit (32-bit 8-element vector indexes over x and dX) */

/*
 * sce_workspace_size -- bytes of device workspace a call with these sizes needs.
 * `bytes` is a HOST pointer. The largest piece is the [T, P] logits buffer
 * (reused in place for its gradient): T * round_up(P or V, 8) elements of dtype.
 * Returns SCE_EINVAL for sizes the call would reject.
 */
SCE_API sce_status sce_workspace_size(int64_t T, int64_t d, int64_t V, int64_t P, int dtype, size_t* bytes);

/*
 * sce_build_candidates -- the candidate build alone ("sampled_softmax.py",
 * CandidateBuilder.build and CandidateBuilder._negatives):
 *   1. mark every class that is a target (-1 = no label, ignored);
 *   2. need = P - (distinct targets); when need > 0 walk the window of the sweep
 *      c_k = (k * stride) mod V for k = offset, offset+1, ... (wrapping mod V) of
 *      length draw = min(V, floor(1.7 * need) + 256), and take the first `need`
 *      classes that are not targets, in window order. If the window holds fewer,
 *      take instead every s-th class (ascending) among the classes that are not
 *      targets, s = max(1, free_count div need), the first `need` of them;
 *   3. C = the marked classes in ascending order (exactly P of them);
 *   4. target_pos[t] / prefix_pos[t] = the position in C of the label, -1 when the
 *      label is -1 or (prefix only) not in C. Prefix targets never enter C.
 *
 *   targets        [T] int64: class id or -1.
 *   prefix_targets [T] int64 or NULL (= every token has no prefix target).
 *   P              1..V (P = 0 is not a candidate build and is rejected here).
 *   stride         gcd(stride mod V, V) must be 1.
 *   offset         sweep index where the window starts; any int64, taken mod V.
 *   candidates_out [P] int32, ascending.   vocab_pos_out [V] int32 or NULL.
 *   target_pos_out [T] int32.              prefix_pos_out [T] int32 or NULL.
 *   aux_out        [4] int64 or NULL: {distinct targets, N = labels with
 *                  position >= 0, next offset = (offset + draw) mod V or offset
 *                  when need = 0, SCE_DEV_* bits}.
 * Needs a workspace of at least sce_workspace_size(T, 8, V, P, SCE_F32) bytes
 * (any size query with the same T, V, P is enough).
 */
SCE_API sce_status sce_build_candidates(const int64_t* targets, const int64_t* prefix_targets, int64_t T,
                                int64_t V, int64_t P, int64_t stride, int64_t offset,
                                int32_t* candidates_out, int32_t* vocab_pos_out,
                                int32_t* target_pos_out, int32_t* prefix_pos_out,
                                int64_t* aux_out, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * sce_build_candidates_host -- the candidate build of sce_build_candidates on the host, for
 * a caller that builds the next microbatch's set on a CPU thread while the GPU runs the
 * current step and uploads it for sampled_ce_forward_backward_prebuilt, the way
 * "sampled_softmax.py" does (CandidateBuilder runs with no device work on a worker thread;
 * SampledSoftmax.prefetch / upload). Same arguments and results as sce_build_candidates,
 * but every pointer is a HOST pointer, nothing is enqueued, and the call returns when the
 * set is built. Device-detected conditions of the device build are reported the same way
 * in aux_out[3] (which may be NULL). No workspace; the call allocates nothing and keeps no
 * state, so calls from different threads are independent. V <= SCE_MAX_V_SAMPLED.
 */
SCE_API sce_status sce_build_candidates_host(const int64_t* targets, const int64_t* prefix_targets,
                                             int64_t T, int64_t V, int64_t P, int64_t stride,
                                             int64_t offset, int32_t* candidates_out,
                                             int32_t* target_pos_out, int32_t* prefix_pos_out,
                                             int64_t* aux_out);

/*
 * sce_build_candidates_noalloc -- sce_build_candidates with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Arguments, results and error
 * behaviour are those of sce_build_candidates. Its scratch (the counters, the
 * candidate bitmap and per-word prefix counts, and the prefix positions when
 * prefix_pos_out is NULL) lives in one static device array of
 * SCE_NOALLOC_SCRATCH_BYTES bytes per GPU, loaded with the library and held until the
 * process ends; the call allocates and frees nothing. The first call on a device looks
 * up that device's copy of the array (with that device current).
 *   Returns SCE_EWORKSPACE, before enqueuing anything, when the sizes need more scratch
 *   than the array holds: about 37 KB of fixed pieces for V <= SCE_MAX_V_SAMPLED, plus
 *   4 * T bytes when prefix_pos_out is NULL (so T up to about 250000 then; any T when
 *   prefix_pos_out is given).
 *   Every call on a GPU uses that GPU's one array, which keeps the last call's
 *   contents (each call rewrites what it reads): calls that overlap in time on one GPU
 *   (other streams, other threads) race and give wrong results. Order them.
 */
#define SCE_NOALLOC_SCRATCH_BYTES (1 << 20)
SCE_API sce_status sce_build_candidates_noalloc(const int64_t* targets,
                                                const int64_t* prefix_targets, int64_t T,
                                                int64_t V, int64_t P, int64_t stride,
                                                int64_t offset, int32_t* candidates_out,
                                                int32_t* vocab_pos_out, int32_t* target_pos_out,
                                                int32_t* prefix_pos_out, int64_t* aux_out,
                                                void* stream);

/*
 * sampled_ce_forward_backward -- the whole step: candidate build (as above),
 * gather W_C = W[C], logits Z = x W_C^T (fp32 accumulation, stored in dtype),
 * per row the log-sum-exp L_t = max_j Z + ln sum_j exp(Z - max), the loss
 *     loss = (1/N) sum_t ( [y'_t >= 0](L_t - Z[t,y'_t]) + [p'_t >= 0](L_t - Z[t,p'_t]) ),
 * with N = the number of labels whose position is >= 0 (targets plus surviving
 * prefix targets; loss = 0 and all gradients 0 when N = 0), the logit gradient
 *     dZ[t,j] = (n_t softmax(Z_t)_j - [j = y'_t] - [j = p'_t]) / N,  n_t = labels of row t,
 * written in place over Z, then dX = dZ W_C and dW_C = dZ^T x, and the dense
 * dW [V, d] = dW_C scattered to the rows of C, exactly zero elsewhere.
 * (Softmax and its gradient: "Learning Triton one kernel at a time: softmax",
 * definition, max subtraction, online softmax and backward sections; the
 * normaliser N counts non-ignored labels as in "16_optimization_checks.py",
 * lm_gradient.) P = 0 runs the same chain over all V classes with no candidate
 * build, gather or scatter; P = V gives bit-identical results to P = 0.
 *
 *   x [T, d], W [V, d]            dtype, d a multiple of 8.
 *   targets, prefix_targets       as in sce_build_candidates.
 *   loss [1] float32.
 *   dX [T, d], dW [V, d]          dtype, overwritten.
 *   candidates_out [P] int32 or NULL; target_pos_out, prefix_pos_out [T] int32 or NULL.
 *   row_lse_out [T] float32 or NULL: L_t.  row_loss_out [T] float32 or NULL: the
 *   row's loss terms before division by N.
 *   aux_out [4] int64 or NULL: as in sce_build_candidates (for P = 0: distinct
 *   targets, or -1 when V > SCE_MAX_V_SAMPLED, then N, offset mod V, SCE_DEV_* bits).
 *   workspace: at least sce_workspace_size(T, d, V, P, dtype) bytes, 256-byte aligned.
 * Inputs x, W, targets and prefix_targets are only read.
 */
SCE_API sce_status sampled_ce_forward_backward(const void* x, const void* W, const int64_t* targets,
                                       const int64_t* prefix_targets, int64_t T, int64_t d,
                                       int64_t V, int64_t P, int64_t stride, int64_t offset,
                                       int dtype, float* loss, void* dX, void* dW,
                                       int32_t* candidates_out, int32_t* target_pos_out,
                                       int32_t* prefix_pos_out, float* row_lse_out,
                                       float* row_loss_out, int64_t* aux_out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * sampled_ce_forward_backward_prebuilt -- the same step from a candidate set built
 * beforehand. "sampled_softmax.py" (CandidateBuilder docstring, SampledSoftmax.prefetch /
 * upload / gather) builds the next microbatch's set off the step's critical path (on a
 * worker thread, then uploads it) and only gathers rows in the step. Here the results of
 * sce_build_candidates (or sce_build_candidates_noalloc, or sce_build_candidates_host
 * uploaded to the device) are the inputs, so a caller can run the next microbatch's build
 * on another stream or a host thread, with its own buffers, while this step runs. The results are bit-identical to
 * sampled_ce_forward_backward on the labels the set was built from.
 *
 *   x, W, T, d, V, dtype, loss, dX, dW, row_lse_out, row_loss_out: as in
 *   sampled_ce_forward_backward (P >= 1 here: a sampled candidate set).
 *   candidates  [P] int32: the set, strictly ascending classes in [0, V).
 *   target_pos  [T] int32 in [-1, P); prefix_pos [T] int32 or NULL (= all -1).
 *   build_aux   [4] int64 or NULL: the build's aux_out; its distinct count, next offset
 *               and device bits are passed on.
 *   aux_out     [4] int64 or NULL: {distinct (build_aux[0], or -1), N counted here from
 *               the positions, next offset (build_aux[2], or -1), SCE_DEV_* bits}.
 *   workspace   as for sampled_ce_forward_backward with the same sizes.
 * The inputs are only read, and must not change until the step has run (stream order).
 * A class out of range or out of order, or a position outside [-1, P), sets
 * SCE_DEV_LABEL_RANGE; every access stays in bounds.
 */
SCE_API sce_status sampled_ce_forward_backward_prebuilt(const void* x, const void* W,
                                                        const int32_t* candidates,
                                                        const int32_t* target_pos,
                                                        const int32_t* prefix_pos,
                                                        const int64_t* build_aux, int64_t T,
                                                        int64_t d, int64_t V, int64_t P,
                                                        int dtype, float* loss, void* dX,
                                                        void* dW, float* row_lse_out,
                                                        float* row_loss_out, int64_t* aux_out,
                                                        void* workspace, size_t workspace_bytes,
                                                        void* stream);

/*
 * sampled_ce_forward_backward_fp8 -- the same step with e4m3 (OCP E4M3, "e4m3fn")
 * matrix-product operands. "sampled_softmax.py" keeps the lm_head as an e4m3 cache,
 * gathers the candidate rows from it as e4m3 and multiplies with scaled fp8 products
 * (SampledLoss rows / rows_t, SampledSoftmax._gather_rows); the scaling is not on the
 * page, and this entry point takes per-tensor power-of-two scales:
 *   s_x = the smallest power of two with max|x| <= 448 s_x, x8 = e4m3(x / s_x);
 *   Z   = bf16( s_x w_scale (x8 W8_C^T) )                (fp32 accumulation);
 *   L_t, the loss, N and the logit gradient g as in sampled_ce_forward_backward,
 *         computed from these bf16 logits;
 *   s_g = the smallest power of two with n_max / N <= 448 s_g (n_max = 2 when
 *         prefix_targets is given, else 1; every |g| <= n_max / N), g8 = e4m3(g / s_g);
 *   dX  = bf16( s_g w_scale (g8 W8_C) ),  dW_C = s_g s_x (g8^T x8),
 *   dW [V, d] bf16 = dW_C in the rows of C, exactly zero elsewhere.
 * e4m3 encodings round to nearest, ties to even.
 *
 *   x [T, d] bf16, d a multiple of 16.    W8 [V, d] e4m3 codes (the lm_head cache).
 *   w_scale (host) > 0, finite: W ~ w_scale * W8; used when w_scale_dev is NULL.
 *   w_scale_dev (device float, or NULL): the cache's scale read on the device in stream
 *         order (as sce_refresh_e4m3_cache writes it, with no host round trip); then
 *         w_scale is ignored, and a value that is not positive and finite sets
 *         SCE_DEV_SCALE_RANGE in aux_out[3].
 *   targets, prefix_targets, P, stride, offset, loss, the position outputs,
 *   row_lse_out, row_loss_out, aux_out: as in sampled_ce_forward_backward.
 *   dX [T, d], dW [V, d] bf16, overwritten.
 *   scales_out [2] float32 or NULL: {s_x, s_g}.
 *   workspace: at least sce_workspace_size(T, d, V, P, SCE_E4M3) bytes, 256-byte aligned.
 * x non-finite, or with 0 < max|x| < 2^-100, sets SCE_DEV_SCALE_RANGE in aux_out[3].
 */
SCE_API sce_status sampled_ce_forward_backward_fp8(const void* x, const void* W8, float w_scale,
                                           const float* w_scale_dev,
                                           const int64_t* targets, const int64_t* prefix_targets,
                                           int64_t T, int64_t d, int64_t V, int64_t P,
                                           int64_t stride, int64_t offset, float* loss, void* dX,
                                           void* dW, int32_t* candidates_out,
                                           int32_t* target_pos_out, int32_t* prefix_pos_out,
                                           float* row_lse_out, float* row_loss_out,
                                           int64_t* aux_out, float* scales_out, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * sampled_ce_forward_backward_fp8_prebuilt -- the e4m3 step from a candidate set built
 * before, the page's own arrangement ("sampled_softmax.py": the set is built on a CPU
 * worker and staged to the GPU, SampledSoftmax; the lm_head is the e4m3 cache). The
 * same results as sampled_ce_forward_backward_fp8 given the same set, bit for bit.
 *   x, W8, w_scale, w_scale_dev, T, d, V, loss, dX, dW, row_lse_out, row_loss_out,
 *   aux_out, scales_out, workspace (sce_workspace_size(T, d, V, P, SCE_E4M3)), stream:
 *         as in sampled_ce_forward_backward_fp8.
 *   candidates, target_pos, prefix_pos, build_aux, P (>= 1): as in
 *         sampled_ce_forward_backward_prebuilt (device memory, validated on the device;
 *         prefix_pos NULL: no prefix targets, n_max = 1).
 */
SCE_API sce_status sampled_ce_forward_backward_fp8_prebuilt(
    const void* x, const void* W8, float w_scale, const float* w_scale_dev,
    const int32_t* candidates, const int32_t* target_pos, const int32_t* prefix_pos,
    const int64_t* build_aux, int64_t T, int64_t d, int64_t V, int64_t P, float* loss, void* dX,
    void* dW, float* row_lse_out, float* row_loss_out, int64_t* aux_out, float* scales_out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sampled_ce_forward_backward_fp8_bf16w -- the e4m3 step from the bf16 weights, with the
 * cache refresh folded in: the step reads only the candidate rows of the e4m3 lm_head
 * cache ("sampled_softmax.py" refreshes the cache, then gathers those rows), so it forms
 * the cache's scale and the codes of exactly those rows itself. max|W| is taken by spare
 * workgroups beside the candidate build, and the row gather reads W[C] in bf16 and
 * writes their codes under the rule of sce_refresh_e4m3_cache:
 *   s_w = float32(max|W| / 448) (1 when W is all zeros), W8_C = e4m3(float32(W[C] / s_w)).
 * The results equal, bit for bit, sce_refresh_e4m3_cache(W) followed by
 * sampled_ce_forward_backward_fp8 with the refreshed cache and its device scale.
 *   W [V, d] bf16 (the lm_head weights, 16-byte aligned); every other argument as in
 *   sampled_ce_forward_backward_fp8, except:
 *   scales_out [3] float32 or NULL: {s_x, s_g, s_w}.
 *   workspace: at least sce_workspace_size(T, d, V, P, SCE_E4M3_BF16W) bytes.
 * A non-finite W sets SCE_DEV_SCALE_RANGE (s_w is then 1).
 */
SCE_API sce_status sampled_ce_forward_backward_fp8_bf16w(
    const void* x, const void* W, const int64_t* targets, const int64_t* prefix_targets, int64_t T,
    int64_t d, int64_t V, int64_t P, int64_t stride, int64_t offset, float* loss, void* dX,
    void* dW, int32_t* candidates_out, int32_t* target_pos_out, int32_t* prefix_pos_out,
    float* row_lse_out, float* row_loss_out, int64_t* aux_out, float* scales_out, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * sce_refresh_e4m3_cache -- rebuilds the e4m3 lm_head cache the fp8 step reads from the
 * bf16 weights ("sampled_softmax.py" refreshes this cache before it gathers candidate
 * rows; the page does not give the encoding). Per-tensor scale, the largest magnitude
 * mapped to e4m3's largest finite value 448:
 *   s_w = float32( max|W| / 448 )  (1 when W is all zeros),
 *   W8  = e4m3( float32(W / s_w) ) (correctly rounded float32 quotient, then round to
 *         nearest even: the codes of torch's float8_e4m3fn cast of that quotient).
 *   W [V, d] bf16 (device), d a multiple of 16, 16-byte aligned; V <= SCE_MAX_V.
 *   W8_out [V, d] e4m3 codes (device, 16-byte aligned), overwritten.
 *   w_scale_out: one device float, overwritten with s_w; pass it to the fp8 step as
 *         w_scale_dev so that the step needs no host round trip.
 *   status_out: one device int32 or NULL; 0, or SCE_DEV_SCALE_RANGE when W holds a
 *         non-finite value (s_w is then 1 and the codes are unspecified).
 *   workspace: at least SCE_REFRESH_WORKSPACE_BYTES of device memory, 256-byte aligned.
 * Two kernels on `stream`; nothing is allocated and no host synchronisation happens.
 */
#define SCE_REFRESH_WORKSPACE_BYTES 8192
SCE_API sce_status sce_refresh_e4m3_cache(const void* W, int64_t V, int64_t d, void* W8_out,
                                          float* w_scale_out, int32_t* status_out,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * sce_ce_rows -- the fused cross-entropy forward/backward of the step on its own, in
 * place over a caller's logits ("Learning Triton one kernel at a time: softmax":
 * row maximum, online (max, sum) merge, softmax gradient; "sampled_softmax.py"
 * docstring and "16_optimization_checks.py" lm_gradient for the labels and N):
 *   for each row t of Z [T, ldz] with columns [0, P) valid,
 *     L_t        = max_j Z_tj + ln sum_j exp(Z_tj - max_j Z_tj)
 *     row loss_t = [y_t >= 0] (L_t - Z_t,y_t) + [p_t >= 0] (L_t - Z_t,p_t)
 *     Z_tj      <- (n_t exp(Z_tj - L_t) - [j = y_t] - [j = p_t]) / N
 *   with y_t = target_pos[t], p_t = prefix_pos[t], n_t = [y_t >= 0] + [p_t >= 0],
 *   N = sum_t n_t (counted on the device) and loss = sum_t row loss_t / N (0 when N = 0).
 *
 *   Z           [T, ldz] dtype, P <= ldz, ldz % 8 == 0, 16-byte aligned; overwritten
 *               (columns [P, ldz) receive zeros).
 *   target_pos  [T] int32 in [-1, P).    prefix_pos [T] int32 or NULL (= all -1).
 *   loss [1] float32.  row_loss_out, row_lse_out [T] float32 or NULL.
 *   aux_out [4] int64 or NULL: {0, N, 0, SCE_DEV_* bits}. A position outside [-1, P)
 *   sets SCE_DEV_LABEL_RANGE and is treated as -1.
 *   workspace  at least sce_ce_rows_workspace_size(T) bytes, 256-byte aligned.
 */
SCE_API sce_status sce_ce_rows_workspace_size(int64_t T, size_t* bytes);
SCE_API sce_status sce_ce_rows(void* Z, int64_t ldz, int64_t T, int64_t P, int dtype,
                               const int32_t* target_pos, const int32_t* prefix_pos, float* loss,
                               float* row_loss_out, float* row_lse_out, int64_t* aux_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * sce_gather_rows -- the row gather of the step on its own ("sampled_softmax.py",
 * SampledSoftmax._gather_rows): out[i, 0:d] = W[idx[i], 0:d] for i < n, bit for bit.
 *   W [V, d] dtype row-major, 16-byte aligned, d % 8 == 0.
 *   idx [n] int32. An index outside [0, V) gives a row of zeros and, when status_out
 *   is not NULL, ORs SCE_DEV_LABEL_RANGE into *status_out (a device int32 the caller
 *   clears beforehand).
 *   out [n, ld_out] dtype, ld_out >= d, ld_out % 8 == 0, 16-byte aligned; columns
 *   [d, ld_out) are not written.
 * No workspace; enqueued on `stream`.
 */
SCE_API sce_status sce_gather_rows(const void* W, int64_t V, int64_t d, const int32_t* idx,
                                   int64_t n, int dtype, void* out, int64_t ld_out,
                                   int32_t* status_out, void* stream);

/*
 * Stage timing for benchmarks. sce_profile_enable(1) creates the HIP events it
 * needs on the current device (once; the only resources the library ever creates,
 * kept until the process ends) and makes every later call of the step entry points
 * record one of them on its stream at each stage boundary (up to 512 calls; later
 * calls are not timed); sce_profile_enable(0) stops it. A step call itself creates
 * nothing. sce_profile_collect waits for the recorded events, writes into stage_ms
 * (HOST array of at least SCE_NUM_STAGES doubles) the milliseconds each stage took
 * summed over the timed calls, stores the number of calls in *ncalls (HOST, may be
 * NULL) and forgets them. Process-wide state: enable and collect must not run
 * concurrently with each other or with timed calls.
 */
enum {
  SCE_STAGE_CANDIDATES = 0, /* candidate build, label remap and the row gather of W[C] */
  SCE_STAGE_LOGITS = 1,
  SCE_STAGE_CE = 2, /* CE forward/backward + loss reduction */
  SCE_STAGE_DX = 3,
  SCE_STAGE_DX_REDUCE = 4, /* sum of the dX k-split partials (empty when dX is not split) */
  SCE_STAGE_DW = 5,
  SCE_STAGE_SCATTER = 6,
  SCE_NUM_STAGES = 7
};
SCE_API sce_status sce_profile_enable(int on);
SCE_API sce_status sce_profile_collect(double* stage_ms, int nstages, int* ncalls);

/* Human-readable name of an sce_status value (static string, never NULL). */
SCE_API const char* sce_status_string(int status);

/* ABI version of this header: 2. */
SCE_API int sce_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAMPLED_CE_H */
