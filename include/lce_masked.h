/*
 * lce_masked.h — C ABI of the MI355X (gfx950) masked cross-entropy library.
 *
 * Two layers, both sum-reduced masked cross-entropy over a large vocabulary:
 *
 *   1. Chunked CE over materialised bf16 logits (ce_chunked_*). Defined by NeMo Automodel
 *      PR #2996, "feat(loss): chunked masked CE, packing-mask preservation, scoped MoE AC":
 *      the first commit message (forward = per-row fp32 logsumexp and label-logit gather
 *      summed into one scalar; backward = softmax recomputed, minus one-hot, times
 *      1/num_label_tokens; zero num_label_tokens guard), the fourth commit message (the
 *      gradient is written into the logits storage) and the *Motivation* section (the fp32
 *      working set is bounded by one [chunk_size, V] slice).
 *
 *   2. Fused linear CE (flce_*): logits z = hidden · weightᵀ (+ bias) never kept in full; the
 *      call returns the loss, grad_hidden, an fp32 grad_weight and grad_bias. Defined by
 *      Liger-Kernel issue #533, "Gradient checkpointing for grad_weight in LFCE" (feature
 *      pitch: per-chunk logits GEMM, grad_weight += (logits gradient)ᵀ · input chunk; the
 *      comments on a fully recomputed variant) and Liger-Kernel issue #941, "No gain in VRAM
 *      usage with LigerFusedLinearCrossEntropyLoss" (inputs: hidden, targets, lm_head weight,
 *      optional bias; the lm_head weight may be tied to the embedding, hence the accumulate
 *      flag).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library never allocates,
 *     frees or synchronises: it validates arguments on the host, enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and returns.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *   - Labels are int32. A row carries a label when label != ignore_index and
 *     0 <= label < V. Any other label that is not ignore_index sets bit
 *     LCE_STATUS_BAD_LABEL in *status_out (device int32, may be NULL) and the row is treated
 *     as ignored; nothing is ever read out of bounds.
 *   - num_label_tokens (T): >= 0 uses that value as the normaliser; < 0 counts the rows that
 *     carry a label, on the device. s = 1/T, and T == 0 gives loss 0 and all-zero gradients
 *     (never NaN).
 *   - grad_output: device pointer to one fp32 upstream gradient g, or NULL for g = 1.
 *     Every gradient is g · s · (softmax − onehot) propagated through the op.
 *   - loss_out: device fp32 scalar, = s · Σ_{labelled rows} (lse_i − z_{i,y_i}); the sum is
 *     taken in fp64 in a fixed order, so results are bitwise repeatable run to run and do not
 *     depend on chunk_size.
 *   - workspace: caller-provided device memory of at least the size the matching
 *     *_workspace_size query returns (256-byte aligned). Its contents on entry do not
 *     matter. Calls that share a workspace must be ordered on one stream.
 *   - Return value: LCE_OK or an error code. Argument errors are reported before any device
 *     work is enqueued; LCE_ERR_HIP means a launch failed (the stream state is then the
 *     caller's to inspect).
 *   - Aliasing: every buffer a call writes (its outputs, status_out and the workspace) must be
 *     disjoint from every other buffer of the call, checked on the host from the pointers and
 *     sizes (LCE_ERR_OVERLAP). The one exception is the in-place CE backward, where the
 *     gradient occupies exactly the logits' rows (same pointer, same row stride).
 *
 * Where the signatures differ from the plain interface of the pages (logits, labels,
 * num_label_tokens, chunk_size for the CE; hidden, targets, weight, bias for the fused layer),
 * the additions are optional outputs or device-side conditions: lse_out (the per-row
 * logsumexp, so a backward need not recompute it), status_out (out-of-range labels reported
 * without a host synchronisation), grad_output (the chain rule's upstream factor) and the
 * caller-provided workspace (the library never allocates).
 */
#ifndef LCE_MASKED_H
#define LCE_MASKED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define LCE_OK                   0
#define LCE_ERR_NULL_ARG         1  /* a required pointer is NULL                                 */
#define LCE_ERR_BAD_SHAPE        2  /* n < 0, v < 1, h < 1, ld < v, or a size overflows int64     */
#define LCE_ERR_BAD_CHUNK        3  /* chunk_size <= 0                                            */
#define LCE_ERR_WORKSPACE        4  /* workspace NULL or smaller than the query's answer          */
#define LCE_ERR_HIP              5  /* a HIP call or kernel launch failed                         */
#define LCE_ERR_DEVICE           6  /* the current device is not gfx950                           */
#define LCE_ERR_BAD_FLAGS        7  /* unknown flag bits                                          */
#define LCE_ERR_ALIGNMENT        8  /* a pointer is not aligned to its element size               */
#define LCE_ERR_OVERLAP          9  /* an output (or the workspace) shares bytes with another
                                       buffer of the call, other than the documented in-place
                                       case of the CE backward                                   */
#define LCE_ERR_SCRATCH_LIMIT   10  /* n > LCE_NOALLOC_MAX_ROWS (allocation-free call only)      */

/* bits of *status_out */
#define LCE_STATUS_BAD_LABEL     1  /* some label was neither ignore_index nor in [0, V)          */

/* flce flags */
#define FLCE_RECOMPUTE           1u /* do not store the chunk's logits; recompute the logits
                                       tile by tile for the gradients (the fully recomputed
                                       schedule of Liger-Kernel issue #533's comments)           */
#define FLCE_ACCUMULATE          2u /* add into grad_weight / grad_bias instead of overwriting
                                       (tied embedding and lm_head, Liger-Kernel issue #941)     */
#define FLCE_ACCUMULATE_GRAD_W   FLCE_ACCUMULATE  /* the same flag, under its other name       */

/* Human-readable name of a return code (static storage; never NULL). flce_status_str is the
 * same function under the name the fused layer's callers look for. */
const char* lce_status_str(int status);
const char* flce_status_str(int status);

/* ------------------------------------------------------------------ chunked CE */

/* Workspace bytes needed by ce_chunked_fwd / ce_chunked_bwd* for n rows. NeMo Automodel PR
 * #2996, *Motivation*: the chunked path bounds the fp32 working set by one [chunk_size, V]
 * slice; here it is smaller still. O(n): the CE kernels
 * stream each row through registers and never build an fp32 [chunk_size, V] slice, so the
 * size does not depend on v or chunk_size. Returns LCE_ERR_BAD_SHAPE / LCE_ERR_BAD_CHUNK /
 * LCE_ERR_NULL_ARG on bad input. Host-only; safe without a GPU. */
int ce_chunked_workspace_size(int64_t n, int64_t v, int64_t chunk_size, size_t* bytes);

/* Forward: loss_out = s · Σ_i (lse_i − z_{i,y_i}) over labelled rows. NeMo Automodel PR
 * #2996, first commit message: per-row fp32 logsumexp plus the label-logit gather,
 * accumulated into one scalar divided by num_label_tokens (zero guard: T == 0 gives 0).
 *   logits      bf16 [n, ld] row-major, first v columns used, read only. Rows without a label
 *               are not read.
 *   labels      int32 [n]
 *   chunk_size  rows per loss partial; must be > 0. The per-row terms are combined in one
 *               fixed order whatever its value (results are chunk-size invariant).
 *   lse_out     fp32 [n] or NULL. Receives lse_i = ln Σ_v exp(z_iv) for labelled rows and 0
 *               for the others. Passing it to the backward saves one read of each row.
 *   status_out  device int32 or NULL; overwritten with LCE_STATUS_* bits.
 * n == 0 is valid (loss 0). */
int ce_chunked_fwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                   const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                   int64_t num_label_tokens, float* loss_out, float* lse_out,
                   int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream);

/* Backward, out of place: grad[i, :] = g · s · (softmax(z_i) − onehot(y_i)) for labelled rows,
 * exactly 0 for the others; fp32 math, rounded to bf16 (nearest even). NeMo Automodel PR
 * #2996, first commit message (the softmax recomputed in the backward, minus the one-hot,
 * times 1/num_label_tokens) and seventh commit message (the logits left intact unless the
 * caller opts in to the in-place form).
 *   logits      bf16 [n, ld] (read)
 *   grad        bf16 [n, ldg] (written, first v columns). grad == logits with ldg == ld is the
 *               in-place case; any other overlap of the two ranges is refused
 *               (LCE_ERR_OVERLAP).
 *   lse         fp32 [n] from ce_chunked_fwd, or NULL to recompute each row's logsumexp
 *               (one more read of every labelled row). */
int ce_chunked_bwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                   uint16_t* grad, int64_t ldg, const int32_t* labels, int32_t ignore_index,
                   int64_t chunk_size, int64_t num_label_tokens, const float* grad_output,
                   const float* lse, int32_t* status_out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Backward in place: as ce_chunked_bwd with grad = logits_inout, ldg = ld. The logits are
 * destroyed; rows without a label are overwritten with zeros (fourth commit message of NeMo
 * Automodel PR #2996: the logits storage is reused as the gradient buffer). */
int ce_chunked_bwd_inplace(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                           const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                           int64_t num_label_tokens, const float* grad_output, const float* lse,
                           int32_t* status_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Forward and in-place backward in one call, when the upstream gradient g is known at
 * forward time (NULL grad_output: g = 1). Liger-Kernel issue #533, feature pitch: Liger's
 * fused linear CE already forms the logits gradient inside its chunked forward and only
 * applies it in the backward; this is that schedule for the materialised logits of NeMo
 * Automodel PR #2996 (first and fourth commit messages: the loss and the gradient of
 * ce_chunked_fwd and ce_chunked_bwd_inplace, written into the logits storage).
 *   logits_inout  bf16 [n, ld], first v columns; on return the gradient
 *                 g · s · (softmax − onehot) for labelled rows and exactly 0 for the others.
 *   loss_out      as ce_chunked_fwd.
 *   lse_out       fp32 [n] or NULL, as ce_chunked_fwd.
 * Results are bitwise those of ce_chunked_fwd followed by ce_chunked_bwd_inplace with the
 * same arguments. Rows with v / 8 <= 16384 (at most 16 aligned 8-element vectors per lane of
 * a 1024-thread workgroup; v up to 131079) are read once, held in registers and written once;
 * longer rows take the two passes internally. Workspace: ce_chunked_workspace_size. n == 0 is
 * valid. */
int ce_chunked_fwd_bwd_inplace(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                               const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                               int64_t num_label_tokens, const float* grad_output,
                               float* loss_out, float* lse_out, int32_t* status_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Rows the allocation-free call below can take: its static scratch is a 256-byte header and
 * one fp32 term per row, 256 + 4 · LCE_NOALLOC_MAX_ROWS bytes (4 MiB + 256 B) per GPU. */
#define LCE_NOALLOC_MAX_ROWS 1048576

/* ce_chunked_fwd_bwd_inplace without a workspace argument, for callers that cannot allocate
 * device memory around the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The library keeps the step's O(n) workspace in a static device
 * array of fixed size, one per GPU, held until the process ends; the call itself allocates
 * and frees nothing. Every other argument, every result and every error code is that of
 * ce_chunked_fwd_bwd_inplace (bit for bit the same kernels and values), plus
 * LCE_ERR_SCRATCH_LIMIT when n > LCE_NOALLOC_MAX_ROWS. All calls on one GPU share its array:
 * calls that may run at the same time on one GPU (different streams, or different host
 * threads without ordering) race on it and must be serialised by the caller; calls ordered
 * on one stream are safe. */
int ce_chunked_fwd_bwd_inplace_noalloc(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                                       const int32_t* labels, int32_t ignore_index,
                                       int64_t chunk_size, int64_t num_label_tokens,
                                       const float* grad_output, float* loss_out,
                                       float* lse_out, int32_t* status_out, void* stream);

/* Unreduced loss (the per-row terms before the sum of NeMo Automodel PR #2996, first commit
 * message; a framework's reduction="none"). No normaliser T is involved.
 * ce_rows_fwd: row_loss_out fp32 [n] receives lse_i − z_{i,y_i} for labelled rows and 0 for
 *   the others; lse_out (fp32 [n] or NULL) as ce_chunked_fwd.
 * ce_rows_bwd: grad[i, :] = grad_rows[i] · (softmax(z_i) − onehot(y_i)) for labelled rows,
 *   exactly 0 for the others (grad_rows: fp32 [n], the upstream gradient of each row's term);
 *   grad == logits with ldg == ld is the in-place case; lse as ce_chunked_bwd.
 * chunk_size is validated as in ce_chunked_fwd and has no other effect. Workspace:
 * ce_chunked_workspace_size. n == 0 is valid. */
int ce_rows_fwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld, const int32_t* labels,
                int32_t ignore_index, int64_t chunk_size, float* row_loss_out, float* lse_out,
                int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream);
int ce_rows_bwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld, uint16_t* grad,
                int64_t ldg, const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                const float* grad_rows, const float* lse, int32_t* status_out, void* workspace,
                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ fused linear CE */

/* Workspace bytes for flce_fwd_bwd, flce_fwd and flce_bwd (NeMo Automodel PR #2996,
 * *Motivation*, for the one-slice bound; Liger-Kernel issue #941, the reply that sizes a
 * chunk's fp32 logits as rows · V · 4 bytes): one fp32 [C, V] logits slice,
 * C = min(chunk_size, n), rows padded to a multiple of 64 columns. The fp32 working set of
 * one chunk is that slice (NeMo Automodel PR #2996, Motivation), and with h a multiple of 64
 * and C >= 64 it is the whole workspace: the call's other state (lse, loss terms, per-tile
 * (max, sum) pairs, label count, sorted labels) then lives in parts of the slice the
 * schedule leaves free, or in rows of grad_hidden before the call writes them. In that
 * layout two chunks share the slice and grad_weight is formed once per two chunks: the
 * stored-logits schedule keeps each chunk's logits as 16-bit values (fp16 of z minus the
 * row's maximum over a 256-column tile); the recomputing schedule (and flce_bwd) keeps each
 * chunk's bf16 probabilities, when grad_hidden is asked for and grad_bias is not. When the
 * stored-logits schedule overwrites grad_weight (no FLCE_ACCUMULATE), chunk_size is a
 * multiple of 64 and the batch is short enough (about n <= 2h), every row's bf16
 * probabilities are kept at once, transposed, in the slice and in grad_weight's own bytes,
 * and grad_hidden and grad_weight are each formed by products over the whole batch (the
 * fp32 working set is still the one slice). Otherwise a few words per chunk row sit beside
 * the slice (lse, label logit, loss term and one (max, sum) pair per 256-column tile);
 * nothing grows with n. Host-only; safe without a GPU. */
int flce_workspace_size(int64_t n, int64_t h, int64_t v, int64_t chunk_size, uint32_t flags,
                        size_t* bytes);

/* Fused linear CE forward + backward in one call, one chunk of rows at a time. Liger-Kernel
 * issue #533, feature pitch (per chunk: logits = input · weightᵀ, the CE gradient of those
 * logits, grad_input, and grad_weight += gradientᵀ · input) and comments (the fully
 * recomputed variant: FLCE_RECOMPUTE); Liger-Kernel issue #941, the opening post (the loss
 * takes hidden states, targets, the lm_head weight and an optional bias; the lm_head weight
 * may be tied to the embedding, which FLCE_ACCUMULATE serves).
 *   hidden       bf16 [n, h] row-major            weight  bf16 [v, h] row-major
 *   bias         fp32 [v] or NULL                 labels  int32 [n]
 *   loss_out     fp32 scalar (required)
 *   lse_out      fp32 [n] or NULL (logsumexp of labelled rows; 0 for the others)
 *   grad_hidden  bf16 [n, h] or NULL: g·s·(P − Y)·W per row, 0 for rows without a label
 *   grad_weight  fp32 [v, h] or NULL: g·s·(P − Y)ᵀ·hidden (+= with FLCE_ACCUMULATE)
 *   grad_bias    fp32 [v] or NULL (needs bias): g·s·Σ_rows (P − Y) (+= with FLCE_ACCUMULATE)
 * where P is the row softmax of z = hidden·weightᵀ + bias and Y the one-hot labels.
 * h must be a multiple of 8 (16-byte rows). Matrix products run on bf16 MFMA with fp32
 * accumulation; the probabilities enter the gradient products as bf16, the one-hot term and
 * the scale g·s are applied in fp32. Where the logits are kept as 16-bit shifted values (see
 * flce_workspace_size) a probability also carries the fp16 rounding of its shifted logit,
 * a relative error of at most exp(2^-11 · (max_v z − z)) − 1; lse and loss always come from
 * the fp32 logits. The loss adds the rows' terms in row order in fp64, so it does not
 * depend on chunk_size.
 * grad_hidden also serves as scratch before its rows are written, and so does grad_weight
 * when it is overwritten (see flce_workspace_size): their contents are defined only once
 * the call has run, and a grad_hidden that overlaps any other buffer of the call (hidden
 * included: there is no in-place form) is refused with LCE_ERR_OVERLAP. */
int flce_fwd_bwd(const uint16_t* hidden, const uint16_t* weight, const float* bias,
                 const int32_t* labels, int64_t n, int64_t h, int64_t v, int32_t ignore_index,
                 int64_t chunk_size, int64_t num_label_tokens, uint32_t flags,
                 const float* grad_output, float* loss_out, float* lse_out,
                 uint16_t* grad_hidden, float* grad_weight, float* grad_bias,
                 int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream);

/* Split form of flce_fwd_bwd for callers that run the loss in a forward pass and the
 * gradients in a later backward pass (Liger-Kernel issue #533, feature pitch and comments:
 * keeping a [V, H] grad_weight alive from forward to backward is what a fully recomputed
 * variant avoids). Between the two calls only lse [n] (fp32, 4·n bytes) has to be kept.
 *
 * flce_fwd: loss_out and lse_out (both required; lse_out [n] receives the logsumexp of each
 * labelled row, 0 for the others). With h a multiple of 64 the logits are reduced inside the
 * logits GEMM and never stored; otherwise they pass through the workspace slice. No
 * gradients; the workspace is sized by flce_workspace_size(n, h, v, chunk_size, 0). */
int flce_fwd(const uint16_t* hidden, const uint16_t* weight, const float* bias,
             const int32_t* labels, int64_t n, int64_t h, int64_t v, int32_t ignore_index,
             int64_t chunk_size, int64_t num_label_tokens, float* loss_out, float* lse_out,
             int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream);

/* flce_bwd: the gradients of flce_fwd_bwd from flce_fwd's lse (same hidden, weight, bias,
 * labels, ignore_index and num_label_tokens): per chunk the logits are recomputed and turned
 * into bf16 probabilities with the given lse, then grad_hidden / grad_weight / grad_bias as
 * in flce_fwd_bwd (any may be NULL; grad_bias needs bias). flags: FLCE_ACCUMULATE only
 * (FLCE_RECOMPUTE is implied and rejected with LCE_ERR_BAD_FLAGS). No loss. grad_hidden and
 * grad_weight equal flce_fwd_bwd's bit for bit; grad_bias is summed in another order when
 * h is a multiple of 64. */
int flce_bwd(const uint16_t* hidden, const uint16_t* weight, const float* bias,
             const int32_t* labels, const float* lse, int64_t n, int64_t h, int64_t v,
             int32_t ignore_index, int64_t chunk_size, int64_t num_label_tokens, uint32_t flags,
             const float* grad_output, uint16_t* grad_hidden, float* grad_weight,
             float* grad_bias, int32_t* status_out, void* workspace, size_t workspace_bytes,
             void* stream);

/* ------------------------------------------------------------------ measurement aid */

/* Opt-in launch timing. While enabled, every kernel the library enqueues is bracketed by a
 * pair of hipEvents recorded on the caller's stream (a few microseconds per launch; off by
 * default; process-wide). Always returns LCE_OK. */
int lce_timing_enable(int enable);

/* Waits for the recorded event pairs, writes up to max_kernels rows (kernel name in static
 * storage, total milliseconds, number of launches) for the kernels timed since the previous
 * read, then resets the totals. *count_out receives the number of kernels seen, which may
 * exceed max_kernels. LCE_ERR_NULL_ARG if count_out is NULL, or max_kernels > 0 and an
 * output array is NULL; LCE_ERR_HIP if an event could not be read. */
int lce_timing_read(int max_kernels, const char** names, double* total_ms, long long* launches,
                    int* count_out);

#ifdef __cplusplus
}
#endif

#endif /* LCE_MASKED_H */
