/*
 * kdkl.h -- fused, chunked top-K KL distillation loss on AMD Instinct MI355X (gfx950).
 *
 * The operation is the "fused chunked KL loss" of "Efficient Knowledge
 * Distillation for LLMs: Offline Top-K Logits and a Fused Chunked KL Loss":
 * the student's vocabulary output projection joined to the loss calculation and
 * processed one sequence chunk at a time, so that the full tokens-by-vocabulary
 * logit tensor is never materialised (thorstenmeyerai.com article, TL;DR and
 * infographic "Fuse and chunk"; aimodeling.com article, "Second cut").  The
 * pages' autograd form recomputes each chunk's logits during backpropagation
 * (infographic "Recompute backward"): kd_chunked_kl_bwd does that.  The one-call
 * kd_chunked_kl_fwd_bwd runs each chunk's backward right after its forward and
 * takes dz from the exponentials that forward kept for that chunk instead.  The teacher is
 * a cache of its top-K tokens and their probabilities per position
 * (aimodeling.com article, "First cut": top-100 probabilities per token).
 *
 * For tokens n = 0..N-1 with hidden state h[n,:] and teacher entries
 * (idx[n,k], p[n,k]), k = 0..K-1:
 *
 *   z[n,v]   = sum_j h[n,j] * W[v,j]                    student logits
 *   lse[n]   = log sum_v exp z[n,v]
 *   l[n]     = sum_k p[n,k] * (log p[n,k] - (z[n,idx[n,k]] - lse[n]))   (0 log 0 = 0)
 *   loss     = sum_n mask[n] * l[n] / count,   count = #{n : mask[n] != 0}
 *
 * and the closed-form gradient of the legiblepapers.com summary
 * (Cross-Examination & FAQs, Q5: a dense M*softmax term minus the sparse teacher
 * correction at the top-K support positions):
 *
 *   dz[n,v]  = (mask[n]/count) * (M[n]*softmax(z[n,:])[v] - sum_{k: idx[n,k]=v} p[n,k]),
 *   M[n]     = sum_k p[n,k],   dh = dz @ W,   dW = dz^T @ h.
 *
 * p is used as given (no renormalisation; M may be below 1); there is no term
 * for the teacher mass outside the top K; temperature is 1.  With count == 0
 * the loss, dh and dW are all zero.
 *
 * Memory: every pointer argument is owned by the caller; the library never
 * allocates or frees device memory.  Scratch space is a caller-provided device
 * workspace whose size depends on min(chunk, N), d, V and K but not otherwise on
 * N, so peak device memory is linear in N.
 */
#ifndef KDKL_H
#define KDKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of h, W and dh. */
typedef enum { KD_F32 = 0, KD_BF16 = 1 } kd_dtype;

/* Return codes. */
typedef enum {
  KD_OK = 0,
  KD_E_ARG = 1,          /* null pointer, bad size or alignment; nothing enqueued     */
  KD_E_INDEX = 2,        /* a teacher index outside [0,V), or a probability that is
                            negative, NaN or infinite; no output written             */
  KD_E_WORKSPACE = 3,    /* workspace smaller than kd_workspace_bytes_group(.., 0, ..);
                            nothing done */
  KD_E_UNSUPPORTED = 4,  /* valid but unsupported shape (d not a multiple of 8, ...)  */
  KD_E_HIP = 5           /* a HIP runtime call failed; outputs undefined              */
} kd_status;

/*
 * kd_workspace_bytes -- device workspace for kd_chunked_kl_fwd_bwd at full speed.
 *
 * Same size arguments as the main call.  Writes the byte count to *bytes_out.
 * Pure host computation (no GPU use).  Returns KD_OK, KD_E_ARG or
 * KD_E_UNSUPPORTED under the same rules as kd_chunked_kl_fwd_bwd.
 * Equal to kd_workspace_bytes_group with dw_group_tokens = 16384.
 */
int kd_workspace_bytes(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                       int32_t dtype, size_t *bytes_out);

/*
 * kd_workspace_bytes_group -- device workspace when the dW accumulation runs over
 * groups of at most dw_group_tokens tokens.
 *
 * In bfloat16, dL/dW is accumulated in float32 by one GEMM per group of chunks, and
 * each such GEMM reads and writes the whole of dW.  The workspace holds a
 * token-contiguous copy of the group's bf16 dz and h: (V + d) * 2 bytes per token of
 * the group (V rounded up to 768).  The group is min(dw_group_tokens, 16384) rounded
 * down to whole chunks, at least one chunk and at most the batch; float32 always uses
 * one chunk.  dw_group_tokens = 0 gives the smallest workspace the calls accept: then no
 * buffer holds more than one chunk's logits.
 * The computing calls (kd_chunked_kl_fwd_bwd, _fwd, _bwd, kd_vocab_shard_fwd, _bwd)
 * take the largest group, up to 16384 tokens, that the workspace passed to them
 * holds, so the caller trades memory for speed by the size it passes; results then
 * differ from the full-size schedule only in float rounding order.
 * Returns KD_E_ARG for a negative dw_group_tokens, otherwise as kd_workspace_bytes.
 */
int kd_workspace_bytes_group(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                             int32_t dtype, int64_t dw_group_tokens, size_t *bytes_out);

/*
 * kd_chunked_kl_fwd_bwd -- loss, dL/dh and dL/dW in one call.
 *
 * Device pointers (all caller-owned, row-major, contiguous):
 *   h         [N, d]  dtype           student hidden states (16-byte aligned)
 *   W         [V, d]  dtype           output projection (16-byte aligned)
 *   topk_idx  [N, K]  int32           teacher token indices
 *   topk_p    [N, K]  float32         teacher probabilities
 *   loss_mask [N]     uint8           nonzero = token counts; NULL = every token counts
 *   loss      [1]     float32         mean loss over counted tokens (written)
 *   dh        [N, d]  dtype           dL/dh, overwritten; rounded once to dtype (RNE)
 *   dW        [V, d]  float32         dL/dW, overwritten (16-byte aligned)
 *   row_loss  [N]     float32         optional: mask[n] ? l[n] : 0     (NULL = skip)
 *   row_lse   [N]     float32         optional: lse[n]                 (NULL = skip)
 *   zg        [N, K]  float32         optional: z[n, idx[n,k]]         (NULL = skip)
 *   workspace         256-byte aligned; kd_workspace_bytes(...) bytes for full speed,
 *                     at least kd_workspace_bytes_group(..., 0, ...) bytes
 * Sizes: N >= 0, 1 <= K <= 32768, V >= 1, d >= 8 with d % 8 == 0, chunk >= 1,
 *   d <= 2^20, V <= 2^24, N*d and N*K below 2^62 (else KD_E_ARG or KD_E_UNSUPPORTED);
 *   one chunk, min(chunk, N) rows, at most 2^22 rows and 2^31 - 1 teacher entries
 *   (else KD_E_UNSUPPORTED).  N == 0 writes loss = 0 and dW = 0.
 * Repeated indices within a row are valid, so K may exceed V: each entry's logit is
 *   gathered on its own and the probabilities of equal indices add up in dz (the
 *   sparse term is a scatter-add).  Each index must lie in [0, V).
 * chunk is the number of token rows whose logits are live at once; the last
 *   chunk may be partial; results do not depend on it beyond float rounding.
 *   Each chunk's backward runs right after its forward, while the chunk's logits
 *   (kept as exp(z - max) in the workspace) are still live, so this call needs no
 *   second logits GEMM; kd_chunked_kl_bwd, which runs after the whole forward,
 *   recomputes them.
 * stream: a hipStream_t (NULL = the null stream).  All work is enqueued on it.
 *   The call synchronises the stream once, after validating the teacher entries
 *   and counting the mask; the rest is asynchronous and the outputs are ready when
 *   the stream's work completes.  Calls sharing one workspace must not overlap;
 *   calls from different host threads with their own workspaces and outputs may run
 *   at the same time, on one stream or on several (the library keeps no device state
 *   between calls, and its host state, the last error, is per thread).
 * Errors: host-side checks run before any device work (KD_E_ARG,
 *   KD_E_UNSUPPORTED, KD_E_WORKSPACE).  Invalid teacher entries give
 *   KD_E_INDEX with no output written.  kd_last_error() describes the failure.
 */
int kd_chunked_kl_fwd_bwd(const void *h, const void *W, int32_t dtype,
                          const int32_t *topk_idx, const float *topk_p,
                          const uint8_t *loss_mask,
                          int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                          float *loss, void *dh, float *dW,
                          float *row_loss, float *row_lse, float *zg,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_chunked_kl_fwd_bwd_async -- kd_chunked_kl_fwd_bwd with no host synchronisation, so
 * that a caller can record it into a HIP graph and replay it (or keep the host ahead of
 * the device).
 *
 * Arguments as kd_chunked_kl_fwd_bwd, plus
 *   status  [1]  int32  device memory, written on the stream after the outputs: KD_OK, or
 *                       KD_E_INDEX when a teacher entry is invalid (an index outside
 *                       [0, V), a probability negative or not finite).
 * With valid entries the outputs equal kd_chunked_kl_fwd_bwd's bit for bit.  With an
 * invalid entry the whole sequence still runs and the outputs are undefined, but no
 * kernel addresses memory outside the arguments and the workspace through it (indices
 * outside the padded vocabulary are skipped).  A mask with no counted token gives loss
 * 0, dh 0 and dW 0 through the same sequence.  The return value covers the host-side
 * checks (KD_E_ARG, KD_E_UNSUPPORTED, KD_E_WORKSPACE, with nothing enqueued) and
 * KD_E_HIP for a failed launch.  Every device operation is a kernel launch on `stream`
 * (no memset or copy), and the sequence depends only on the sizes, the pointers and the
 * workspace size, so a recorded graph replays it for new contents of the same buffers.
 * The kernel timing of kd_profile_enable must be off while recording, and one ordinary
 * call should come first, so that loading the kernels is not part of the recording.
 */
int kd_chunked_kl_fwd_bwd_async(const void *h, const void *W, int32_t dtype,
                                const int32_t *topk_idx, const float *topk_p,
                                const uint8_t *loss_mask,
                                int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                                float *loss, void *dh, float *dW,
                                float *row_loss, float *row_lse, float *zg, int32_t *status,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_chunked_kl_fwd_bwd_f32dh -- kd_chunked_kl_fwd_bwd with dh written in float32.
 *
 * The pages' loss is an autograd function of the hidden states (codewithpapers.app
 * record: _SparseKLHiddenStatesChunkedFunction); its backward receives the upstream
 * gradient g of the loss only after the forward.  A caller that wants the one-call speed
 * in that setting runs this call in its forward (the gradients for g = 1) and
 * kd_scale_grads in its backward.  dh here is [N, d] float32 (16-byte aligned), the
 * float32 sums that kd_chunked_kl_fwd_bwd rounds to dtype; every other argument, output,
 * workspace size, stream behaviour and error as kd_chunked_kl_fwd_bwd, whose loss, dW and
 * row outputs it reproduces bit for bit.
 */
int kd_chunked_kl_fwd_bwd_f32dh(const void *h, const void *W, int32_t dtype,
                                const int32_t *topk_idx, const float *topk_p,
                                const uint8_t *loss_mask,
                                int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                                float *loss, float *dh, float *dW,
                                float *row_loss, float *row_lse, float *zg,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_scale_grads -- apply the upstream gradient g of the loss to gradients computed
 * for g = 1 (by kd_chunked_kl_fwd_bwd_f32dh): by the chain rule dL'/dh = g * dL/dh
 * and dL'/dW = g * dL/dW for L' = g * L.
 *   grad_loss [1]    float32  device   g
 *   dh_f32    [N, d] float32  device   input, 16-byte aligned
 *   dh        [N, d] dtype    device   output: g * dh_f32 rounded once to dtype (RNE);
 *                                      may be dh_f32 itself only when dtype is KD_F32
 *   dW        [V, d] float32  device   scaled in place (left untouched when g == 1, where
 *                                      the product is exact)
 * All work is enqueued on stream; no synchronisation.  Errors: KD_E_ARG for a null
 * required pointer, a misaligned one, an unknown dtype or a negative size.
 */
int kd_scale_grads(const float *grad_loss, const float *dh_f32, void *dh, int32_t dtype,
                   int64_t N, int64_t d, float *dW, int64_t V, void *stream);

/*
 * kd_chunked_kl_fwd -- the forward half: loss and the per-token logsumexp.
 *
 * The loss as a function of the hidden states with the logits recomputed in the
 * backward pass (thorstenmeyerai.com article, infographic "Recompute backward";
 * aimodeling.com article, "Second cut").  Computes exactly the loss, row_loss and zg
 * of kd_chunked_kl_fwd_bwd (bit for bit, on the same inputs and chunk) and writes
 *   row_lse   [N]     float32   lse[n] = log sum_v exp z[n,v]   (required when N > 0)
 * which is the state kd_chunked_kl_bwd reads.  row_loss and zg are optional (NULL =
 * skip).  dh and dW are not computed.  Same sizes, workspace, stream behaviour and
 * errors as kd_chunked_kl_fwd_bwd; it never uses a dW group, so
 * kd_workspace_bytes_group(..., 0, ...) bytes run it at full speed.  N == 0 writes
 * loss = 0.
 */
int kd_chunked_kl_fwd(const void *h, const void *W, int32_t dtype,
                      const int32_t *topk_idx, const float *topk_p,
                      const uint8_t *loss_mask,
                      int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                      float *loss, float *row_lse, float *row_loss, float *zg,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_chunked_kl_bwd -- the backward half: dh and dW for an upstream gradient.
 *
 * Recomputes the logits chunk by chunk from h and W and forms the closed-form
 * gradient of the legiblepapers.com summary (Cross-Examination & FAQs, Q5), scaled by
 * the upstream gradient g = grad_loss[0] of the mean loss:
 *   dz[n,v] = g * (mask[n]/count) * (M[n]*exp(z[n,v] - row_lse[n]) - sum_{k: idx[n,k]=v} p[n,k])
 *   dh = dz @ W  (rounded once to dtype),  dW = dz^T @ h  (float32, overwritten).
 * Inputs as for kd_chunked_kl_fwd_bwd, plus
 *   row_lse   [N]  float32  device   the logsumexp written by kd_chunked_kl_fwd for the
 *                                    same h, W and chunk (required when N > 0)
 *   grad_loss [1]  float32  device   g, read on the device (no host synchronisation)
 * With g = 1 and row_lse from kd_chunked_kl_fwd, dh and dW equal those of
 * kd_chunked_kl_fwd_bwd up to rounding (that call derives dz from its forward's
 * exponentials rather than recomputed logits).  Teacher entries are validated again (one stream
 * synchronisation); count == 0 or N == 0 gives dh = 0 and dW = 0.  Same workspace
 * (kd_workspace_bytes), stream behaviour and errors as kd_chunked_kl_fwd_bwd.
 */
int kd_chunked_kl_bwd(const void *h, const void *W, int32_t dtype,
                      const int32_t *topk_idx, const float *topk_p,
                      const uint8_t *loss_mask,
                      int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                      const float *row_lse, const float *grad_loss,
                      void *dh, float *dW,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Vocabulary shards -- one GPU's share of an output head split over the vocabulary.
 *
 * The pages' implementation takes tensor-parallel rank and size arguments
 * (codewithpapers.app record of the released code: tensor_parallel_rank,
 * tensor_parallel_size); here a shard is W_shard = rows [v_offset, v_offset + V_shard)
 * of a V_total-row W, teacher indices stay global (entries outside the shard are
 * skipped), and the three calls below are what one GPU runs between the collectives:
 *
 * kd_vocab_shard_fwd: per token n, over the shard's logits z[n,v] (v in the shard)
 *   shard_max[n]    = max_v z[n,v]
 *   shard_sumexp[n] = sum_v exp(z[n,v] - shard_max[n])
 *   shard_pz[n]     = sum_{k: idx[n,k] in the shard} p[n,k] * z[n,idx[n,k]]
 *   zg [N,K]        = optional: z at the in-shard entries, 0 elsewhere (NULL = skip)
 *   (these three [N] float32 arrays are what the shards exchange: an all-gather)
 * kd_vocab_shard_combine: from G shards' statistics laid out [G][N] each,
 *   row_lse[n] = M + log sum_g shard_sumexp[g,n] exp(shard_max[g,n] - M), M = max_g,
 *   l[n] = sum_k p log p - sum_g shard_pz[g,n] + (sum_k p) row_lse[n],
 *   loss = sum_n mask[n] l[n] / count; row_loss[n] = mask[n] ? l[n] : 0 (optional).
 *   Workspace: kd_vocab_shard_combine_workspace_bytes(N).  No host synchronisation: the
 *   count divides the loss on the device.
 * kd_vocab_shard_bwd: with the global row_lse and the upstream gradient g
 *   (grad_loss[0], on the device), for v in the shard
 *   dz[n,v] = g (mask[n]/count) (M[n] exp(z[n,v] - row_lse[n]) - sum_{k: idx=v} p[n,k]),
 *   dh_partial [N,d] float32 = dz @ W_shard  (the shards' partials are summed: an
 *                              all-reduce; then rounded to dtype by the caller),
 *   dW_shard [V_shard,d] float32 = dz^T @ h  (overwritten).
 * Sizes, dtypes, alignment, workspace (kd_workspace_bytes with V = V_shard), stream
 * behaviour and errors as kd_chunked_kl_fwd_bwd; teacher indices are checked against
 * [0, V_total) and v_offset + V_shard <= V_total <= 2^24.  With G = 1 and the whole
 * vocabulary as the shard, the three calls give the loss, dh and dW of
 * kd_chunked_kl_fwd_bwd up to float rounding.
 */
int kd_vocab_shard_fwd(const void *h, const void *W_shard, int32_t dtype,
                       const int32_t *topk_idx, const float *topk_p,
                       int64_t N, int64_t d, int64_t V_shard, int64_t v_offset,
                       int64_t V_total, int32_t K, int64_t chunk,
                       float *shard_max, float *shard_sumexp, float *shard_pz, float *zg,
                       void *workspace, size_t workspace_bytes, void *stream);
int kd_vocab_shard_combine_workspace_bytes(int64_t N, size_t *bytes_out);
int kd_vocab_shard_combine(const float *shard_max, const float *shard_sumexp,
                           const float *shard_pz, int32_t G, const float *topk_p,
                           const uint8_t *loss_mask, int64_t N, int32_t K, float *loss,
                           float *row_lse, float *row_loss,
                           void *workspace, size_t workspace_bytes, void *stream);
int kd_vocab_shard_bwd(const void *h, const void *W_shard, int32_t dtype,
                       const int32_t *topk_idx, const float *topk_p,
                       const uint8_t *loss_mask,
                       int64_t N, int64_t d, int64_t V_shard, int64_t v_offset,
                       int64_t V_total, int32_t K, int64_t chunk,
                       const float *row_lse, const float *grad_loss,
                       float *dh_partial, float *dW_shard,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_teacher_topk -- the teacher top-K cache producer.
 *
 * The offline step that runs the teacher once and keeps, per position, its most
 * likely tokens with their scores (thorstenmeyerai.com article, TL;DR and
 * infographic "Select top 100", "Write cache"), as the probabilities the loss
 * reads (aimodeling.com article, "First cut").  For every row n of teacher logits:
 *   row_lse[n]    = log sum_v exp t[n,v]                      (optional, NULL = skip)
 *   topk_idx[n,k] = the K tokens with the largest logits, in decreasing order of
 *                   logit; equal logits in increasing token order (+0.0 == -0.0)
 *   topk_p[n,k]   = exp(t[n, topk_idx[n,k]] - row_lse[n])  (full-softmax
 *                   probability; the K values are not renormalised)
 * Device pointers, caller-owned, row-major:
 *   logits   [N, V]  dtype (KD_BF16 or KD_F32), aligned to its element size
 *   topk_idx [N, K]  int32;  topk_p [N, K] float32;  row_lse [N] float32 or NULL
 *   workspace        >= kd_topk_workspace_bytes() bytes, 256-byte aligned
 * Sizes: N >= 0, 1 <= K <= min(V, 256), V < 2^29, N < 2^31.
 * Each row is read from device memory once.  The call synchronises the stream once,
 * at the end, to read the validity flag: a row with a NaN or +inf logit, or with no
 * finite logit, gives KD_E_INDEX and the outputs are undefined.  Other errors are
 * host-side checks made before any device work.
 */
int kd_topk_workspace_bytes(size_t *bytes_out);
int kd_teacher_topk(const void *logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
                    int32_t *topk_idx, float *topk_p, float *row_lse,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * kd_teacher_topk_noalloc -- kd_teacher_topk for callers that cannot allocate device
 * memory (tight serving loops, harnesses that forbid hipMalloc): no workspace argument
 * and no allocation of any kind.  Like kd_teacher_topk it synchronises its stream once
 * to report bad rows, so it cannot be recorded into a HIP graph.
 *
 * The 256-byte workspace of kd_teacher_topk (one validity flag) is replaced by a
 * static module array of 256 bytes that every device the library runs on holds from
 * module load until the process ends.  Its address on the current device is looked up
 * once per device (hipGetSymbolAddress) on that device's first call; the flag is
 * cleared by a fill kernel at the start of every call.  Every size the allocating
 * call accepts fits, so no size is rejected for the scratch; arguments, outputs,
 * results (bit for bit), limits, stream behaviour and errors are kd_teacher_topk's.
 * The current device must be the one that logits, the outputs and stream belong to.
 * All calls on one device share its array: calls that overlap on one device (other
 * threads, other streams) race on the flag, so they must be serialised by the caller.
 */
int kd_teacher_topk_noalloc(const void *logits, int32_t dtype, int64_t N, int64_t V,
                            int32_t K, int32_t *topk_idx, float *topk_p, float *row_lse,
                            void *stream);

/* Text describing the last non-OK return on the calling thread ("" if none). */
const char *kd_last_error(void);

/* Library interface version: 5 (it increments when a call is added or changes). */
int kd_version(void);

/*
 * Kernel timing for measurement.  While enabled, the library records a pair of
 * HIP events on the call's stream around every launch and files it under the
 * launch's kernel class.  kd_profile_read waits for the recorded events, adds
 * their durations into *total_ms and *launches for the class, and clears them.
 * Classes are numbered 0 .. kd_profile_num_classes()-1; kd_profile_class_name
 * names them.  Not thread-safe; meant for benchmarks.
 */
int kd_profile_enable(int on);
int kd_profile_num_classes(void);
const char *kd_profile_class_name(int cls);
int kd_profile_read(int cls, double *total_ms, int64_t *launches);

/*
 * Clock measurement for benchmarks (not part of the loss).  kd_clock_stamp enqueues on
 * `stream` one kernel of n_groups one-wave workgroups; workgroup g writes three words at
 * stamps[3g]: the compute unit it ran on (accelerator complex in bits 35:32, the
 * hardware-id register in bits 31:0, whose bits 15:8 number the unit within it), that
 * unit's shader cycle counter, and the device's constant-rate counter.  With n_groups a
 * few times the number of compute units every unit writes at least one stamp.  Two
 * stamps around some work, paired unit by unit (the cycle counters of different units
 * are not aligned), give each unit's average shader clock over the work: cycles /
 * constant ticks * kd_wall_clock_khz().  stamps: device memory for 3 * n_groups uint64,
 * 8-byte aligned, caller-owned; 1 <= n_groups <= 65536, else KD_E_ARG.
 * kd_wall_clock_khz writes the constant counter's rate in kHz (current device).
 */
int kd_clock_stamp(uint64_t *stamps, int32_t n_groups, void *stream);
int kd_wall_clock_khz(int32_t *khz_out);

#ifdef __cplusplus
}
#endif

#endif /* KDKL_H */
