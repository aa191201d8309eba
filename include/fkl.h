/*
 * fkl.h - C ABI of libfkl: the fused chunked top-K KL distillation loss
 * (forward and backward) on AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * The loss described on the pages "Multiverse Computing ... (iitak.ru)"
 * (third and fifth paragraphs) and "Wissensdestillation mit deutlich weniger
 * GPU-Speicher" (section "KL-Verlust wird in Blöcken berechnet"): the student's
 * output projection is fused into a KL loss against a cached teacher top-K, the
 * sequence is processed in blocks ("chunks") of rows whose logits are never
 * kept, and the backward pass recomputes each block. Temperature handling
 * (logits divided by T before each softmax, KL term scaled by T^2) follows
 * "Дистилляция и сжатие моделей", section "Как это работает: мягкие метки и
 * температура". With z = hidden . W^T (W stored [V, d]):
 *
 *   lse_r      = ln sum_v exp(z_rv / T)
 *   p_rk       = softmax_k(topk_logit_r. / T)        (renormalised over K)
 *   row_loss_r = T^2 sum_k p_rk (ln p_rk - (z_r,idx_rk / T - lse_r))
 *   loss       = sum_r row_loss_r
 *   G_rv       = s T (exp(z_rv / T - lse_r) sum_k p_rk - sum_{k: idx_rk = v} p_rk)
 *   grad_hidden = G . W,   grad_W = H^T . G   (stored [V, d])
 *
 * where s is the upstream gradient of ``loss``. Terms with p_rk = 0 (teacher
 * logit -inf) contribute nothing.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensor arguments are DEVICE pointers to dense row-major arrays. The
 *   caller owns every buffer, including the workspace; the library never
 *   allocates or frees device memory and keeps no state between calls
 *   (re-entrant; concurrent calls must use distinct workspaces and outputs).
 * - Work is enqueued on ``stream`` (a hipStream_t passed as void*; NULL = the
 *   default stream). Calls return without waiting for the GPU, except under
 *   FKL_FLAG_VALIDATE_IDX, which synchronises the stream once.
 * - Arguments are validated before anything is enqueued: a call that returns
 *   an error has written nothing. No exception or abort crosses the ABI.
 *   Device faults surface at the caller's next synchronisation.
 * - Outputs must not alias inputs or each other.
 * - dtype FKL_BF16: hidden, weight and grad_hidden are bf16 (raw 16-bit);
 *   FKL_F32: fp32. Ids are int32; teacher logits, lse, loss, row_loss, topk_z
 *   and grad_weight are fp32 in both modes. Accumulation is fp32.
 * - Shapes: N >= 0 tokens (rows; N = 0 is an empty batch), d >= 8 with
 *   d % 8 == 0, V >= 1, 1 <= K <= min(V, 4096), chunk >= 1 rows per pass (the
 *   result does not depend on it beyond rounding; it bounds the workspace).
 *   Ids must lie in [0, V) (checked only under FKL_FLAG_VALIDATE_IDX; an id
 *   out of range without the flag is undefined behaviour). An id repeated
 *   within a row acts additively: each (id, logit) pair is its own term.
 * - hidden, weight, grad_hidden, grad_weight and workspace must be 16-byte
 *   aligned; the fp32/int32 arrays 4-byte aligned.
 */
#ifndef FKL_H
#define FKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FKL_ABI_VERSION 1

/* status codes */
#define FKL_OK 0            /* success */
#define FKL_E_ARG 1         /* null/misaligned pointer, bad shape, T not finite or <= 0 */
#define FKL_E_UNSUPPORTED 2 /* unknown dtype, d % 8 != 0, K > 4096 */
#define FKL_E_WORKSPACE 3   /* workspace smaller than fkl_workspace_size reports */
#define FKL_E_HIP 4         /* a HIP launch or runtime call failed (text in fkl_last_error) */
#define FKL_E_INDEX 5       /* FKL_FLAG_VALIDATE_IDX: an id outside [0, V) */

/* dtypes of hidden / weight / grad_hidden */
#define FKL_F32 0
#define FKL_BF16 1

/* flags */
#define FKL_FLAG_ACCUMULATE_GRAD_W 1u /* backward adds into grad_weight instead of overwriting */
#define FKL_FLAG_VALIDATE_IDX 2u      /* check ids on the device first (synchronises the stream) */

/* Returns FKL_ABI_VERSION of the loaded library. */
int32_t fkl_abi_version(void);

/* Static text for a status code (never NULL). */
const char* fkl_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). The pointer
 * stays valid until the next fkl_* call on this thread. */
const char* fkl_last_error(void);

/* Workspace bytes needed by fkl_forward and fkl_backward for these shapes
 * (host-only, enqueues nothing). Both grow with chunk * V (the one
 * chunk-sized logit-gradient buffer of the backward) and with N (per-row
 * scratch), never with N * V. Either output pointer may be NULL. */
int32_t fkl_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                           int32_t dtype, size_t* fwd_bytes, size_t* bwd_bytes);

/* Forward pass.
 *   hidden     [N, d]  student final hidden states (dtype)
 *   weight     [V, d]  LM-head weight in nn.Linear layout (dtype)
 *   topk_idx   [N, K]  int32 teacher top-K token ids
 *   topk_logit [N, K]  fp32 teacher logits at those ids
 *   T > 0              temperature;  chunk: rows per pass
 *   flags              0 or FKL_FLAG_VALIDATE_IDX
 * Outputs:
 *   loss       [1]     fp32 sum of row losses (required)
 *   lse        [N]     fp32 ln sum_v exp(z_rv / T) (required; the backward needs it)
 *   row_loss   [N]     fp32 per-row loss (may be NULL)
 *   topk_z     [N, K]  fp32 raw student logits z at the given ids, the same
 *                      values the logit tiles feed the log-sum-exp (may be NULL;
 *                      passing it to fkl_backward saves a recomputation)
 * The N x V logits are never stored: each chunk's logit tiles live only in
 * registers; z at the teacher ids is taken from them as they are formed. */
int32_t fkl_forward(const void* hidden, const void* weight, const int32_t* topk_idx,
                    const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                    int64_t V, int32_t K, int32_t dtype, uint32_t flags, float* loss, float* lse,
                    float* row_loss, float* topk_z, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Backward pass: gradients of s * loss with respect to hidden and weight.
 *   hidden, weight, topk_idx, topk_logit, T, chunk, N, d, V, K, dtype: as in
 *                      the forward (same values)
 *   lse        [N]     from fkl_forward (required)
 *   topk_z     [N, K]  from fkl_forward, or NULL to recompute it (by one dot
 *                      product per id: a different summation order, so the
 *                      gradients then agree with the saved-topk_z ones to
 *                      rounding, not bitwise)
 *   grad_loss  [1]     device fp32 upstream gradient s, or NULL for s = 1
 *   flags              FKL_FLAG_ACCUMULATE_GRAD_W and/or FKL_FLAG_VALIDATE_IDX
 * Outputs:
 *   grad_hidden [N, d] (dtype), overwritten
 *   grad_weight [V, d] fp32, overwritten (or accumulated into)
 * Each chunk's logits are recomputed tile by tile and turned into the logit
 * gradient G; G is held for one chunk only (chunk x V in the workspace) and
 * consumed by the two gradient products. */
int32_t fkl_backward(const void* hidden, const void* weight, const int32_t* topk_idx,
                     const float* topk_logit, const float* lse, const float* topk_z,
                     const float* grad_loss, float T, int64_t chunk, int64_t N, int64_t d,
                     int64_t V, int32_t K, int32_t dtype, uint32_t flags, void* grad_hidden,
                     float* grad_weight, void* workspace, size_t workspace_bytes, void* stream);

/* Forward pass without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments, outputs and results are those
 * of fkl_forward (the same kernels run); the workspace is a static 64 MiB
 * device array of the library instead, one copy per GPU, held from the
 * library's first use on that GPU until the process ends. Its device address
 * is looked up on the first call on each device (hipGetSymbolAddress); the
 * call allocates nothing.
 *   - The shapes must fit: the workspace fkl_workspace_size reports as
 *     fwd_bytes must be at most 64 MiB (N <= 39 168 rows at K = 100,
 *     V = 128 256, chunk = 2048), else FKL_E_WORKSPACE before anything runs.
 *   - stream must belong to the current device (FKL_E_ARG otherwise).
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     behind: calls that overlap on one GPU (concurrent streams, or host
 *     threads) race and give undefined results; calls ordered on one stream
 *     are safe. */
int32_t fkl_forward_noalloc(const void* hidden, const void* weight, const int32_t* topk_idx,
                            const float* topk_logit, float T, int64_t chunk, int64_t N,
                            int64_t d, int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                            float* loss, float* lse, float* row_loss, float* topk_z,
                            void* stream);

/* Loss options
 * ------------
 * The ml-book page ("Дистилляция и сжатие моделей", section "Как это
 * работает: мягкие метки и температура") describes the student's total loss
 * as the KL term plus the ordinary cross-entropy on the true labels; training
 * also needs padding rows masked out and mean reductions. The *_ex entry
 * points take these through a struct (NULL = the plain loss above):
 *
 *   loss = sum_r w_r (a_kl T^2 KL_r + a_ce CE_r),  CE_r = lse1_r - z_r,y_r,
 *   lse1_r = ln sum_v exp(z_rv)   (temperature 1),
 *   a_kl = alpha, a_ce = 1 - alpha with labels; a_kl = 1, a_ce = 0 without.
 *
 * Rows with w_r = 0 contribute nothing (their teacher logits may then all
 * be -inf, e.g. padding). A mean over the valid rows is row_weight = mask /
 * mask.sum(). The gradients follow: G_r = s w_r (a_kl T (softmax_T(z_r) sum_k
 * p_rk - scatter(p_r)) + a_ce (softmax_1(z_r) - onehot(y_r))). */
typedef struct fkl_loss_options {
  const float* row_weight; /* [N] fp32 per-row weights, or NULL (all 1) */
  const int32_t* labels;   /* [N] hard labels in [0, V), a value < 0 for a row
                              without one; or NULL (no cross-entropy term) */
  float alpha;             /* with labels: weight of the KL term (the
                              cross-entropy gets 1 - alpha); finite */
  float* lse1;             /* [N] fp32 ln sum_v exp(z_rv) at temperature 1:
                              written by the forward when non-NULL; read by
                              the backward, which requires it when labels are
                              given and T != 1 (else it may be NULL) */
  const float* teacher_lse; /* [N] fp32 teacher ln sum_v exp(l_rv / T) over the
                              full vocabulary (fkl_teacher_topk_ex can write
                              it), or NULL. Given, the teacher is not
                              renormalised over its K entries: p_k = exp(l_k / T
                              - teacher_lse) and the rest of its mass forms a
                              tail bucket, p_tail = 1 - sum_k p_k, matched by
                              the student's mass outside the cached ids,
                              1 - S with S = sum_k q_(idx_k):
                              KL_r = sum_k p_k ln(p_k / q_k)
                                     + p_tail ln(p_tail / (1 - S)). */
} fkl_loss_options;

/* fkl_forward, fkl_backward, fkl_forward_keep and fkl_backward_keep with loss
 * options (the opts pointer may be NULL). Under FKL_FLAG_VALIDATE_IDX labels
 * >= V are rejected too. row_loss holds the weighted per-row loss. */
int32_t fkl_forward_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                       const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                       int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                       const fkl_loss_options* opts, float* loss, float* lse, float* row_loss,
                       float* topk_z, void* workspace, size_t workspace_bytes, void* stream);
int32_t fkl_backward_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                        const float* topk_logit, const float* lse, const float* topk_z,
                        const float* grad_loss, float T, int64_t chunk, int64_t N, int64_t d,
                        int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                        const fkl_loss_options* opts, void* grad_hidden, float* grad_weight,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Forward-chunked variant ("keep the logits")
 * ------------------------------------------
 * The pages name a less aggressive alternative to the fused method: the loss
 * is still computed chunk by chunk, but the student logits of every chunk are
 * kept for the backward pass, which then needs no recompute. It is faster and
 * needs an N x V buffer ("Wissensdestillation mit deutlich weniger
 * GPU-Speicher", section "KL-Verlust wird in Blöcken berechnet"; the method
 * table of the malakhovai.ru article lists it as the fast variant). These
 * entry points implement it for callers whose memory allows the buffer; the
 * results are those of fkl_forward / fkl_backward up to rounding (the forward
 * outputs are identical; the backward starts from logits rounded to dtype
 * instead of recomputed ones).
 *
 * Kept-logits buffer: N rows of keep_pitch = round_up(V, 64) elements of dtype,
 * row-major; element (r, v) holds z_rv rounded to dtype (bf16: round to
 * nearest even) for v < V and zero for V <= v < keep_pitch. The caller owns it.
 *
 * fkl_keep_sizes: bytes of the kept-logits buffer (N * keep_pitch * element
 * size) and of the fkl_backward_keep workspace (O(N * (K + d)), per-row
 * coefficients and an fp32 grad_hidden accumulator). Host-only. Returns
 * FKL_E_UNSUPPORTED when 256 kept rows exceed 2 GiB (V above about 4 million
 * in bf16). Either output pointer may be NULL. */
int32_t fkl_keep_sizes(int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype,
                       size_t* logits_bytes, size_t* bwd_bytes);

/* fkl_forward plus the kept logits: arguments and outputs as fkl_forward
 * (workspace sized by fkl_workspace_size's fwd_bytes), and
 *   logits [N, keep_pitch] (dtype) written as described above (may be NULL
 *                       only when N = 0)
 *   logits_bytes        its size; FKL_E_WORKSPACE if below fkl_keep_sizes */
int32_t fkl_forward_keep(const void* hidden, const void* weight, const int32_t* topk_idx,
                         const float* topk_logit, float T, int64_t chunk, int64_t N, int64_t d,
                         int64_t V, int32_t K, int32_t dtype, uint32_t flags, float* loss,
                         float* lse, float* row_loss, float* topk_z, void* logits,
                         size_t logits_bytes, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Backward pass from kept logits: arguments and outputs as fkl_backward
 * (there is no chunk: nothing is recomputed), and
 *   logits [N, keep_pitch] as written by fkl_forward_keep with the same
 *                      inputs. It is CONSUMED: the call overwrites it with
 *                      the logit gradient G (dtype), so it serves one
 *                      backward pass only (may be NULL only when N = 0).
 *   workspace          at least fkl_keep_sizes's bwd_bytes
 * G = s T (softmax_T(z) sum_k p_k - scatter(p)) is formed in place row by row
 * (teacher-id entries from topk_z, recomputed when topk_z is NULL), then
 * grad_hidden = G . W in one MFMA product over the whole vocabulary and
 * grad_W = G^T . H in fp32 over row blocks. */
int32_t fkl_backward_keep(const void* hidden, const void* weight, const int32_t* topk_idx,
                          const float* topk_logit, const float* lse, const float* topk_z,
                          const float* grad_loss, float T, int64_t N, int64_t d, int64_t V,
                          int32_t K, int32_t dtype, uint32_t flags, void* logits,
                          size_t logits_bytes, void* grad_hidden, float* grad_weight,
                          void* workspace, size_t workspace_bytes, void* stream);

int32_t fkl_forward_keep_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                            const float* topk_logit, float T, int64_t chunk, int64_t N,
                            int64_t d, int64_t V, int32_t K, int32_t dtype, uint32_t flags,
                            const fkl_loss_options* opts, float* loss, float* lse,
                            float* row_loss, float* topk_z, void* logits, size_t logits_bytes,
                            void* workspace, size_t workspace_bytes, void* stream);
int32_t fkl_backward_keep_ex(const void* hidden, const void* weight, const int32_t* topk_idx,
                             const float* topk_logit, const float* lse, const float* topk_z,
                             const float* grad_loss, float T, int64_t N, int64_t d, int64_t V,
                             int32_t K, int32_t dtype, uint32_t flags,
                             const fkl_loss_options* opts, void* logits, size_t logits_bytes,
                             void* grad_hidden, float* grad_weight, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Teacher top-K cache
 * -------------------
 * The step before the loss: the pages run the teacher once and keep, for
 * every position, its 100 most probable tokens ("Эффективная дистилляция
 * знаний ..." (malakhovai.ru), second paragraph; "Multiverse Computing ...
 * (iitak.ru)", third paragraph; "Wissensdestillation mit deutlich weniger
 * GPU-Speicher", section "Teacher-Ausgaben einmalig zwischenspeichern").
 * With l = hidden . weight^T (teacher final hidden states [N, d], teacher LM
 * head [V, d] in nn.Linear layout, fp32 accumulation), per row r:
 *   topk_idx[r]   the K ids with the largest l_rv, by value descending, ties
 *                 to the lower id (the most probable tokens of the teacher
 *                 softmax at any temperature, in order)
 *   topk_logit[r] l_rv at those ids (fp32, exactly the accumulated values)
 * These are the topk_idx / topk_logit inputs of fkl_forward. Logits must be
 * finite. 1 <= K <= min(V, 1024); other shapes and dtypes as for the loss.
 *
 * fkl_topk_workspace_size: host-only; bytes of one chunk's fp32 logits
 * (V * round_up(min(chunk, N), 64) * 4) plus per-row scratch.
 * fkl_teacher_topk: flags must be 0. Rows are processed `chunk` at a time; the
 * result does not depend on chunk. Rows whose candidate list overflows (more
 * than 2048 logits at or above the K-th largest 128-vocab slice maximum,
 * e.g. massive ties) take an exact but slower path. */
int32_t fkl_topk_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                                int32_t dtype, size_t* bytes);
/* fkl_teacher_topk plus, when teacher_lse is non-NULL, the teacher's
 * full-vocabulary log-sum-exp at temperature T per row, teacher_lse[r] =
 * ln sum_v exp(l_rv / T) (fp32; the tail-bucket input of fkl_loss_options).
 * T must be finite and > 0 when teacher_lse is requested. */
int32_t fkl_teacher_topk_ex(const void* hidden, const void* weight, int64_t N, int64_t d,
                            int64_t V, int32_t K, int64_t chunk, int32_t dtype, uint32_t flags,
                            float T, int32_t* topk_idx, float* topk_logit, float* teacher_lse,
                            void* workspace, size_t workspace_bytes, void* stream);
int32_t fkl_teacher_topk(const void* hidden, const void* weight, int64_t N, int64_t d, int64_t V,
                         int32_t K, int64_t chunk, int32_t dtype, uint32_t flags,
                         int32_t* topk_idx, float* topk_logit, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Student-renormalised top-K loss: an alternative reading of how the cache's
 * tail is treated, which the pages leave open (the cache itself:
 * "Multiverse Computing ... (iitak.ru)", third paragraph; "Wissensdestillation
 * mit deutlich weniger GPU-Speicher", section "Teacher-Ausgaben einmalig
 * zwischenspeichern"; softening by T and the T^2 factor: "Дистилляция и
 * сжатие моделей", section "Как это работает: мягкие метки и температура").
 * Teacher and student are both softened by T and renormalised over the K
 * cached entries of the row, so only the student's logits at the cached ids
 * enter: no vocabulary-wide log-sum-exp and no vocabulary GEMM. Per row r,
 * over the entries with a finite teacher logit (a -inf entry is padding and
 * takes part in neither softmax):
 *   p_k = softmax_k(l_rk / T),  q_k = softmax_k(z_r,idx_rk / T)
 *   row_loss_r = w_r T^2 sum_k p_k (ln p_k - ln q_k),  loss = sum_r row_loss_r
 *   dloss/dz_r,idx_rk = s w_r T (q_k sum_j p_j - p_k)
 * with w_r = row_weight[r] (1 when row_weight is NULL; a row of weight 0
 * contributes nothing, whatever its logits) and s = *grad_loss (1 when NULL).
 * A row of nonzero weight without a finite teacher logit contributes 0.
 * Shapes and dtypes as fkl_forward / fkl_backward (hidden [N, d] and the
 * weight [V, d] in dtype, ids int32 [N, K] in [0, V) on every entry, padding
 * included; teacher logits fp32 [N, K]); K <= 1024, d <= 8192,
 * N * K < 2^31 (FKL_E_UNSUPPORTED otherwise). Duplicate ids inside a row act
 * as separate entries. No chunk parameter: the work and the workspace are
 * O(N * K * (1 + d / K)) and O(V) and never touch N x V.
 *
 * fkl_renorm_workspace_size: bytes of the forward and backward workspaces
 *   (either pointer may be NULL). The backward workspace holds the K
 *   coefficients per row, a counting sort of the N * K (row, entry) pairs by
 *   id (at most 256 MiB of per-block counters; the sorted rows, ids and
 *   coefficients), a copy of the hidden rows in slices of 64 columns
 *   (N * ceil(d / 64) * 64 elements of dtype), chunk partials of grad_W, and
 *   for the (at most 2048) ids with the most pairs a dense coefficient matrix
 *   (at most 256 MiB) with its product's output copies.
 * fkl_renorm_forward: writes loss[0] and, when non-NULL, row_loss [N] and
 *   topk_z [N, K] (the student logit at each cached id, fp32 dot product of
 *   the hidden row and the weight row). flags: 0 or FKL_FLAG_VALIDATE_IDX.
 * fkl_renorm_backward: grad_hidden [N, d] in dtype (overwritten) and
 *   grad_weight [V, d] fp32 (overwritten; added to under
 *   FKL_FLAG_ACCUMULATE_GRAD_W). topk_z from the forward may be passed to skip
 *   the gather (NULL: recomputed). grad_W is summed without float atomics in
 *   a fixed order, so repeated calls give the same bits.
 * Alignment, ownership, stream and error behaviour as for fkl_forward /
 * fkl_backward; outputs must not alias inputs. */
int32_t fkl_renorm_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype,
                                  size_t* fwd_bytes, size_t* bwd_bytes);
int32_t fkl_renorm_forward(const void* hidden, const void* weight, const int32_t* topk_idx,
                           const float* topk_logit, float T, int64_t N, int64_t d, int64_t V,
                           int32_t K, int32_t dtype, uint32_t flags, const float* row_weight,
                           float* loss, float* row_loss, float* topk_z, void* workspace,
                           size_t workspace_bytes, void* stream);
int32_t fkl_renorm_backward(const void* hidden, const void* weight, const int32_t* topk_idx,
                            const float* topk_logit, const float* topk_z, const float* grad_loss,
                            float T, int64_t N, int64_t d, int64_t V, int32_t K, int32_t dtype,
                            uint32_t flags, const float* row_weight, void* grad_hidden,
                            float* grad_weight, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Per-kernel timing, a profiling aid (off by default). While enabled, every
 * kernel launch the library makes is bracketed by two HIP events recorded on
 * the launch stream; the events cost a few microseconds of GPU time each.
 * Kernel ids run from 0 to fkl_kernel_count() - 1.
 *   fkl_timing_enable: on = 1 enables, 0 disables; returns the previous state.
 *   fkl_timing_reset:  waits for outstanding events and zeroes all totals.
 *   fkl_timing_read:   waits for outstanding events (host-blocking) and writes
 *                      the launch count and summed milliseconds of one kernel
 *                      since the last reset; FKL_E_ARG for an unknown id.
 *   fkl_kernel_name:   static name of a kernel id, NULL if unknown.
 * Timing state is process-wide; concurrent library calls on several streams
 * are timed correctly but share the totals. */
int32_t fkl_timing_enable(int32_t on);
int32_t fkl_timing_reset(void);
int32_t fkl_timing_read(int32_t kernel, int64_t* launches, double* total_ms);
int32_t fkl_kernel_count(void);
const char* fkl_kernel_name(int32_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* FKL_H */
