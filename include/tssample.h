/*
 * tssample.h -- C ABI of the MI355X (gfx950) batched token sampler.
 *
 * One call samples one token id per output row from a logits matrix
 * [rows_in_buffer, vocab] and (optionally) returns the log-prob of that id
 * under the processed distribution.  The operation is the one described by
 *   - "core.inference.sampling.base" (Megatron-Core API docs), class Sampling,
 *     methods sample_kernel (gather_indices, token_to_request_index, n rows of
 *     a [>=n, vocab] logits tensor, returns ids [n]) and sample_speculative
 *     (decode requests contribute 1 + num_speculative_tokens rows, prefill
 *     requests 1 row);
 *   - "core.inference.sampling.flashinfer_sampling" (Megatron-Core API docs),
 *     class FlashInferSampling: per-step top-p-only / top-k-only / joint
 *     dispatch from CPU-side flags no_top_k / no_top_p (no GPU sync), seeded
 *     Philox randomness that advances per step, caller-owned output [n], and
 *     log_probs_kernel (log-probs of the processed distribution);
 *   - the TokenSpeed Triton sampling backend source page: per-request pools of
 *     temperature / top_k / top_p / 64-bit seed, Gumbel-max sampling, int32
 *     index arrays.
 *
 * Per output row r (0 <= r < n):
 *   src = gather_indices ? gather_indices[r] : r      row of the logits buffer
 *   q   = token_to_request_index ? token_to_request_index[r] : r   parameter slot
 *   x   = logits[src, 0:vocab] (NaN read as -inf, -0 as +0)
 *   K   = top-k set: the first min(k, #finite) indices in the order
 *         (x descending, index ascending) when 1 <= k < vocab, else all finite
 *   s   = x / temperature[q]  (temperature < 1e-5 means greedy: first index of
 *         that order, log-prob 0)
 *   P   = top-p set inside K: j is kept when the softmax(s)-mass over K of the
 *         members with a strictly larger logit is below p; p >= 1 - 1e-6 keeps
 *         all of K; the top tie group is always kept
 *   g_j = -ln(-ln u_j), u_j = ((w_j >> 9) + 1/2) * 2^-23, w_j = word (j & 3) of
 *         Philox4x32-10(key = seed[q], counter = (j >> 2, r, off lo, off hi))
 *         with off = step_offset (+ step_offsets[q] when given), mod 2^64
 *         (Salmon et al., SC'11)
 *   id  = argmax over P of s_j + g_j (smallest j on exact ties)
 *   lp  = s_id - logsumexp over P of s
 * A row whose entries are all -inf/NaN yields id -1 and lp NaN.
 *
 * Conventions shared by every entry point:
 *   - Pointers named "device" are device memory of the sampler's GPU; the
 *     caller owns every buffer.  The library never allocates inside ts_sample /
 *     ts_log_probs.
 *   - "stream" is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work and return without synchronising; results are valid once the stream
 *     has reached them.  A sampler handle may be used from one host thread at
 *     a time.
 *   - Errors are returned as ts_status, never thrown.  Host-checkable argument
 *     errors are detected before any work is enqueued.  Gather and request
 *     indices inside device arrays are read without a guard (an out-of-range
 *     one is undefined behaviour); a caller that does not trust them checks
 *     them first with ts_check_indices, which writes a device error word.
 *     Token ids are guarded: one outside [0, vocab) has a defined result
 *     (ts_log_probs, ts_raw_log_probs_at).
 */
#ifndef TSSAMPLE_H
#define TSSAMPLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ts_status {
  TS_OK = 0,
  TS_E_ARG = 1,    /* null pointer, negative size or inconsistent argument */
  TS_E_DTYPE = 2,  /* unsupported logits dtype */
  TS_E_SIZE = 3,   /* n above max_rows, stride below vocab, rows_in_buffer below n, ... */
  TS_E_HIP = 4,    /* a HIP runtime call failed (launch, device query, ...) */
  TS_E_NOMEM = 5   /* device memory for the handle's workspace could not be allocated */
} ts_status;

typedef enum ts_dtype {
  TS_F32 = 0,      /* IEEE binary32 logits */
  TS_BF16 = 1      /* bfloat16 logits (upper half of a binary32) */
} ts_dtype;

/* Filter routes chosen on the host from the batch-level flags (no GPU sync):
 * "flashinfer_sampling": dedicated top-p or top-k kernel when only one filter is
 * in use, joint kernel only for mixed batches. */
typedef enum ts_route {
  TS_ROUTE_NONE = 0,   /* no_top_k && no_top_p */
  TS_ROUTE_TOPK = 1,   /* !no_top_k && no_top_p */
  TS_ROUTE_TOPP = 2,   /* no_top_k && !no_top_p */
  TS_ROUTE_JOINT = 3   /* !no_top_k && !no_top_p */
} ts_route;

typedef struct ts_sampler ts_sampler;

/* Per-request sampling parameters, structure of arrays, device memory, indexed
 * by the request slot q.  top_k may be NULL when the call passes no_top_k = 1 and
 * top_p may be NULL when it passes no_top_p = 1: the flags are promises that no
 * row uses that filter, and the route then never reads the array. */
typedef struct ts_params {
  const float* temperature;   /* [num_requests] */
  const int32_t* top_k;       /* [num_requests]; k <= 0 or k >= vocab: filter off */
  const float* top_p;         /* [num_requests]; p >= 1 - 1e-6: filter off */
  const uint64_t* seed;       /* [num_requests] */
  int32_t num_requests;       /* > 0 */
  /* [num_requests] or NULL.  Per-request Philox offsets, added (mod 2^64) to
   * the call's step_offset: the request-indexed offset pool of the TokenSpeed
   * Triton sampling backend page (`offsets_pool`).  Because the kernels read
   * them from device memory, a call captured in a HIP graph draws fresh noise
   * on each replay once the caller advances them between replays (the
   * "flashinfer_sampling" page explains why a captured sampler with the offset
   * baked in as a constant replays the same random numbers).  Not read by
   * ts_log_probs, which draws no noise. */
  const uint64_t* step_offsets;
} ts_params;

/* Create a sampler for logits rows of `vocab` entries and up to `max_rows`
 * output rows per call on HIP device `device`.  Any device memory the handle
 * needs is allocated here, once; ts_sample / ts_log_probs allocate nothing.
 * device == -1 creates a validation-only handle: its calls run every host-side
 * argument check and then return TS_E_HIP without touching a GPU (useful to
 * test callers on a machine without one).
 * Errors: TS_E_ARG (out == NULL, vocab < 1, vocab >= 2^31, max_rows < 1,
 * device < -1), TS_E_HIP (no such device), TS_E_NOMEM. */
ts_status ts_create(int64_t vocab, int32_t max_rows, int32_t device, ts_sampler** out);

/* Release a sampler (NULL is accepted).  The caller must ensure no enqueued
 * call on it is still running. */
ts_status ts_destroy(ts_sampler* sampler);

/* Sample one id per output row (see the top of this file for the definition).
 *   logits          device, row-major [rows_in_buffer, row_stride] of `dtype`;
 *                   only the first `vocab` entries of a row are read
 *   rows_in_buffer  rows present in `logits` (>= n when gather_indices is NULL)
 *   row_stride      elements between consecutive rows (>= vocab)
 *   n               output rows, 0 <= n <= max_rows (n == 0 enqueues nothing)
 *   gather_indices  device int32 [n] or NULL
 *   token_to_request_index  device int32 [n] or NULL (NULL: q = r, which then
 *                   needs params->num_requests >= n)
 *   params          host struct of device arrays
 *   step_offset     Philox offset of this call (advance it between steps)
 *   no_top_k, no_top_p  batch-level flags (0/1) computed by the caller on the host
 *   out_ids         device int32 [n], written
 *   out_logprob     device float [n] or NULL, written when non-NULL
 *   stream          hipStream_t
 * Errors: TS_E_ARG, TS_E_DTYPE, TS_E_SIZE (host-side checks), TS_E_HIP (launch). */
ts_status ts_sample(ts_sampler* sampler, const void* logits, ts_dtype dtype,
                    int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                    const int32_t* gather_indices, const int32_t* token_to_request_index,
                    const ts_params* params, uint64_t step_offset,
                    int32_t no_top_k, int32_t no_top_p,
                    int32_t* out_ids, float* out_logprob, void* stream);

/* Log-probs of the processed distribution ("flashinfer_sampling",
 * log_probs_kernel): for every output row, lp_j = s_j - logsumexp_P(s) for j in
 * P and -inf outside P (greedy rows: 0 at the greedy id, -inf elsewhere; rows
 * with no finite logit: NaN).  Arguments as for ts_sample, plus
 *   token_ids  device int32 [n] or NULL
 *   out        device float: [n, vocab] row-major when token_ids is NULL, else [n]
 *              holding lp at token_ids[r] (-inf for an id outside [0, vocab)).
 *              Any float alignment is accepted; full
 *              rows into a 16-byte aligned buffer take the kernels that store 16
 *              bytes at a time
 * Errors: as ts_sample. */
ts_status ts_log_probs(ts_sampler* sampler, const void* logits, ts_dtype dtype,
                       int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                       const int32_t* gather_indices, const int32_t* token_to_request_index,
                       const ts_params* params, int32_t no_top_k, int32_t no_top_p,
                       const int32_t* token_ids, float* out, void* stream);

/* Log-probs of the raw logits at given ids: for every output row r,
 *   out[r] = x[src, id] - logsumexp_j x[src, j]  over the whole row,
 * with no temperature and no filter (the selected-token log-probs that the
 * TokenSpeed Triton sampling backend page writes from the logits and the
 * sampled ids).  NaN logits read as -inf; a NaN or -inf entry at id gives
 * -inf; an id outside [0, vocab) or a row with no finite logit gives NaN.
 *   logits, dtype, rows_in_buffer, row_stride, n, gather_indices  as for ts_sample
 *   token_ids   device int32 [n]
 *   out         device float [n], written
 *   stream      hipStream_t
 * Uses the handle's workspace (one call per handle at a time).
 * Errors: TS_E_ARG, TS_E_DTYPE, TS_E_SIZE (host-side checks, or a vocabulary
 * too large for the split kernel: more than 64 * 16384 entries), TS_E_HIP. */
ts_status ts_raw_log_probs_at(ts_sampler* sampler, const void* logits, ts_dtype dtype,
                              int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                              const int32_t* gather_indices, const int32_t* token_ids,
                              float* out, void* stream);

/* Per-row request index of the speculative-verify layout
 * ("core.inference.sampling.base", sample_speculative): decode request d in
 * [0, num_decode) owns rows d*(1+num_spec) .. d*(1+num_spec)+num_spec, prefill
 * request i owns row num_decode*(1+num_spec)+i and has index num_decode+i.
 * Writes n = num_decode*(1+num_spec)+num_prefill entries of out_map (capacity
 * entries available); with on_device != 0 out_map is device memory and the
 * write is enqueued on `stream`, else it is host memory written synchronously.
 * *out_n (host) receives n.
 * Errors: TS_E_ARG (negative counts, NULL pointers), TS_E_SIZE (capacity < n),
 * TS_E_HIP. */
ts_status ts_build_spec_map(int32_t num_decode, int32_t num_prefill, int32_t num_spec,
                            int32_t* out_map, int32_t capacity, int32_t on_device,
                            void* stream, int32_t* out_n);

/* Debug check of the device index arrays of a ts_sample / ts_log_probs call,
 * whose values those calls read through without a guard (see the conventions
 * at the top of this file).  For callers that do not trust them; not part of
 * the pages' operation.
 *   n, gather_indices, rows_in_buffer, token_to_request_index  as for ts_sample
 *                   (either array may be NULL: it is then not checked)
 *   num_requests    the parameter slots (params->num_requests)
 *   error_word      device uint32 [1], written: 0, or TS_INDEX_GATHER_OUT (a
 *                   gather index outside [0, rows_in_buffer)) | TS_INDEX_REQUEST_OUT
 *                   (a request index outside [0, num_requests))
 * Enqueued on `stream` (hipStream_t); no handle, no workspace.
 * Errors: TS_E_ARG (n < 0, error_word NULL, rows_in_buffer < 1 with a gather
 * array, num_requests < 1 with a request array), TS_E_HIP. */
#define TS_INDEX_GATHER_OUT 1u
#define TS_INDEX_REQUEST_OUT 2u
ts_status ts_check_indices(int32_t n, const int32_t* gather_indices, int64_t rows_in_buffer,
                           const int32_t* token_to_request_index, int32_t num_requests,
                           uint32_t* error_word, void* stream);

/* Chain verification of speculative drafts against the target's samples (the
 * verify step of the TokenSpeed Triton sampling backend page,
 * TritonSamplingBackend.verify: one target sample per row of the speculative
 * layout, then each request's draft chain is checked against them; the page
 * names the step and its outputs but not its arithmetic, so this is a reading).
 * Request b in [0, bs) owns rows b*n_per_req .. b*n_per_req + n_per_req - 1.
 *   candidates      device int32 [bs, n_per_req] row-major: column 0 the
 *                   request's last verified token, columns 1.. its drafts
 *   target_sampled  device int32 [bs * n_per_req]: the target's sample per row
 *                   (e.g. ts_sample's out_ids over the decode rows)
 *   predicts        device int32 [bs * n_per_req], written
 *   accept_index    device int32 [bs * n_per_req] ([bs, n_per_req]), written
 *   accept_length   device int32 [bs], written
 * Draft i+1 of request b is accepted while every earlier draft was and it
 * equals target_sampled[b*n_per_req + i]; accept_length[b] counts the accepted
 * drafts (0 .. n_per_req-1), so a request emits accept_length[b] + 1 tokens.
 * Positions i = 0 .. accept_length[b] get predicts = target_sampled[b*n+i] and
 * accept_index = b*n + i; every other position gets -1 in both.  Buffers are
 * caller-owned and must not overlap; the call is enqueued on `stream`
 * (hipStream_t) and needs no handle and no workspace.
 * Errors: TS_E_ARG (bs < 0, n_per_req < 1, a NULL pointer with bs > 0),
 * TS_E_SIZE (bs * n_per_req > 2^31 - 1), TS_E_HIP. */
ts_status ts_verify_chain(int32_t bs, int32_t n_per_req, const int32_t* candidates,
                          const int32_t* target_sampled, int32_t* predicts,
                          int32_t* accept_index, int32_t* accept_length, void* stream);

/* Largest n that ts_sample_noalloc accepts. */
#define TS_NOALLOC_MAX_ROWS 1024

/* ts_sample without a handle and without any device allocation, for callers
 * that cannot call hipMalloc: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments and results as
 * ts_sample (the sampler's vocabulary is passed as `vocab`), on the current
 * HIP device.  The scratch memory the kernels need (split-row tickets and
 * partial results, the top-p route's per-row state and cutoff lists; about
 * 4.2 MB) is a
 * fixed-size device array inside the library: each GPU the library runs on
 * holds its own copy until the process ends.  The first call on a device
 * looks up that copy's address and clears its tickets with a small kernel on
 * `stream`; later calls find them at zero again, because every call leaves
 * them so.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (two streams, or two host threads) race and may return wrong
 * results; serialise them.  Inputs and outputs are the caller's, as for
 * ts_sample; nothing is allocated or freed here.
 * Errors: TS_E_ARG, TS_E_DTYPE, TS_E_SIZE (n > TS_NOALLOC_MAX_ROWS, and the
 * checks of ts_sample), TS_E_HIP. */
ts_status ts_sample_noalloc(int64_t vocab, const void* logits, ts_dtype dtype,
                            int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                            const int32_t* gather_indices, const int32_t* token_to_request_index,
                            const ts_params* params, uint64_t step_offset,
                            int32_t no_top_k, int32_t no_top_p,
                            int32_t* out_ids, float* out_logprob, void* stream);

/* Vocabulary mask, applied to the logits in place before sampling (the
 * TokenSpeed Triton sampling backend page applies a vocab_mask to the logits
 * after its NaN guard and before the greedy or Gumbel step; the mask's body is
 * not printed there).  For every row r of the buffer (0 <= r < rows) with mask
 * row m = mask_index ? mask_index[r] : r, entry j < vocab keeps its logit when
 * bit (j mod 32) of mask[m * mask_stride_words + j / 32] is 1 and is set to
 * -inf when it is 0; entries past vocab (a padded row_stride) are not touched.
 * Every route then treats a masked entry as any other -inf entry (never
 * sampled; a row left with no finite entry yields id -1 and lp NaN).
 *   vocab              entries per row
 *   logits             device bf16 or fp32 [rows, row_stride], modified in place
 *   dtype              TS_BF16 or TS_F32
 *   rows, row_stride   rows to mask, elements between rows (>= vocab)
 *   mask               device uint32 [mask rows, mask_stride_words]
 *   mask_stride_words  words between mask rows (>= ceil(vocab / 32))
 *   mask_index         device int32 [rows] or NULL (then mask row r for row r;
 *                      with it, e.g. one mask per request for speculative rows)
 *   stream             hipStream_t
 * Needs no handle and allocates nothing.  Errors: TS_E_ARG (vocab < 1 or
 * >= 2^31, rows < 0, NULL logits or mask with rows > 0), TS_E_DTYPE,
 * TS_E_SIZE (row_stride < vocab, mask_stride_words < ceil(vocab / 32)),
 * TS_E_HIP. */
ts_status ts_apply_vocab_mask(int64_t vocab, void* logits, ts_dtype dtype, int64_t rows,
                              int64_t row_stride, const uint32_t* mask, int64_t mask_stride_words,
                              const int32_t* mask_index, void* stream);

/* The route the flags select (pure host function, no GPU). */
ts_route ts_select_route(int32_t no_top_k, int32_t no_top_p);

/* Static text for a status code. */
const char* ts_status_str(ts_status status);

#ifdef __cplusplus
}
#endif

#endif /* TSSAMPLE_H */
