/*
 * spec_verify.h -- C ABI of the batched speculative-decoding verifier
 * (lossless rejection sampler) for AMD Instinct MI355X (gfx950).
 *
 * The operation is the verify step defined on the spec-decoding page at
 * dpshk.com/news/5598276 (scraped title "企业官网建设流程全解析"):
 *
 *   section 3.1  for every request b and draft position i the target model
 *                supplies logits for gamma_b + 1 positions; p = softmax(l / T);
 *                draft token x_i (drawn by the draft model from q_i) is
 *                accepted with probability min(1, p_i(x_i) / q_i(x_i));
 *                verification stops at the first rejection;
 *   section 3.2  the rejected position is redrawn from the residual
 *                (p - q)_+ / sum (p - q)_+, which makes the emitted tokens
 *                distributed exactly as p;
 *   section 5.2  q is floored at 1e-10 before dividing, the test is the strict
 *                comparison of the uniform with the accept probability, and acceptance is a
 *                prefix property (a cumulative product of the accept bits);
 *   section 5.3  when all gamma_b drafts are accepted a bonus token is drawn
 *                from the (gamma_b + 1)-th target distribution;
 *   section 5.4  the number of accepted drafts is what the caller uses to
 *                truncate its KV cache;
 *   section 8    draft and target share one vocabulary (pitfall 1); T = 0 is
 *                greedy decoding (pitfall 2).
 *
 * Readings where the page is silent (fixed here, identical in the CPU oracle):
 *   - T_b <= 0 or NaN selects the greedy variant: g_i = argmax of the raw
 *     logits (lowest id on ties); x_i is accepted iff x_i == g_i; the token
 *     at the first mismatch (or the bonus position) is g.  q and the uniforms
 *     are not read for such requests.
 *   - The uniforms are an input, [B, gamma + 2] fp32 in [0, 1): columns
 *     0 .. gamma_b - 1 drive the accept tests, column gamma the residual draw,
 *     column gamma + 1 the bonus draw (gamma = the padded width below).
 *   - A draft made without a draft model (prompt lookup, page section 7)
 *     proposes x_i with certainty: q_i is the point mass at x_i, so x_i is
 *     accepted with probability p_i(x_i) and the residual is p_i with x_i
 *     removed.  A sparse q (top-k (id, prob) lists) is the same q stored
 *     without its zeros.
 *   - A draw with weights w and uniform v returns min{x : C_x > v * S} where
 *     C_x is the running sum of w in ascending token id and S = C_{V-1}
 *     (zero-weight tokens are never returned).  If rounding leaves the
 *     residual with S <= 0, the draw uses p instead.
 *
 * All entry points are plain C: device buffers are raw device pointers owned by
 * the caller, sizes are integers, and the stream is an opaque hipStream_t
 * (NULL = the legacy default stream).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum sv_status {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1,    /* a host-visible argument violates the contract */
    SV_ERR_OUT_OF_MEMORY = 2,  /* device allocation failed in spec_verify_create */
    SV_ERR_DEVICE = 3,         /* a HIP call failed (launch, event, copy) */
    SV_ERR_UNSUPPORTED = 4,    /* dtype / size outside what the library handles */
    SV_ERR_CAPACITY = 5,       /* batch, gamma or vocab exceed the context's limits */
    SV_ERR_DEVICE_CONTRACT = 6 /* an earlier call on this context broke the device-side
                                  contract (see sv_device_error); nothing was enqueued.
                                  Read and clear the bits with spec_verify_device_errors */
};

/* Logits element type. */
enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 };

/* Context flags. */
enum sv_flags {
    SV_FLAG_PROFILE = 1u,      /* record per-kernel HIP events (see spec_verify_profile_read) */
    SV_FLAG_TWO_KERNEL = 2u    /* schedule: rows kernel, then draw kernel (also the default) */
};

/* Device-side contract violations, OR-ed into a sticky per-context word.  A
 * request that breaks the contract gets -1 in every token column and in
 * num_accepted, is not counted in the acceptance counters, and no access
 * leaves the buffers' bounds.  Once the device has run such a call, every
 * later spec_verify_run on the context returns SV_ERR_DEVICE_CONTRACT until
 * spec_verify_device_errors clears the word. */
enum sv_device_error {
    SV_DEVERR_DRAFT_ID = 1u,   /* a draft id outside [0, vocab) (the page's section 8, pitfall 1:
                                  draft and target share one vocabulary) */
    SV_DEVERR_OFFSETS = 2u,    /* draft_offsets not prefix sums with 0 <= gamma_b <= gamma and
                                  offsets[batch] <= total_draft: requests whose own offsets are
                                  inconsistent get -1; other requests whose rows those offsets
                                  misplace are unspecified */
    SV_DEVERR_NONFINITE = 4u,  /* a sampled target row without a positive finite normaliser (no
                                  finite logit, NaN or +inf logits) */
    SV_DEVERR_TOPK = 16u       /* sparse q: an entry id outside [-1, vocab), or the drafted token
                                  listed twice in its row */
};

/* Largest number of (id, prob) entries per draft row of a sparse q. */
#define SV_MAX_TOPK 64

/* Acceptance counters (optional sv_args.stats, uint32, accumulated with
 * device-scope atomics and never cleared by the library; the caller zeroes
 * them when it wants a fresh count).  For a call with padded width gamma:
 *   [0]                         requests verified
 *   [1]                         drafts proposed (sum of gamma_b)
 *   [2]                         drafts accepted (sum of num_accepted)
 *   [3]                         requests with every draft accepted (a bonus token)
 *   [4 + k], k = 0..gamma       requests with num_accepted == k
 *   [5 + gamma + i], i < gamma  requests whose draft i was tested (i < gamma_b, i <= k)
 *   [5 + 2 gamma + i]           requests whose draft i was accepted (i < k)
 * They feed acceptance-rate monitoring (the spec-decoding page's section 6.2
 * log of acceptance rate and accepted tokens per step) without a host copy of
 * the outputs. */
#define SV_STATS_LEN(gamma) (5 + 3 * (gamma))

/* Limits fixed at creation.  max_gamma <= SV_MAX_GAMMA. */
#define SV_MAX_GAMMA 128
typedef struct sv_config {
    int32_t max_batch;     /* largest batch passed to run, >= 1 */
    int32_t max_gamma;     /* largest padded draft width, 0 .. SV_MAX_GAMMA */
    int32_t vocab;         /* V, shared by draft and target (page section 8, pitfall 1), 1 .. 524288 */
    int32_t logits_dtype;  /* SV_F32 or SV_BF16 */
    uint32_t flags;        /* SV_FLAG_* */
} sv_config;

/*
 * One verify step.  Layout (row-major, contiguous, device memory):
 *   request b owns gamma_b = off[b+1] - off[b] drafts, where off = draft_offsets
 *   (prefix sums, off[0] = 0, off[batch] = total_draft) or, when draft_offsets is
 *   NULL, gamma_b = gamma for every b and off[b] = b * gamma.
 *   target_logits  [total_draft + batch, vocab]  logits_dtype; request b's rows
 *                  are off[b] + b .. off[b] + b + gamma_b (the last one is the
 *                  bonus position).  Rows must be aligned to the element size.
 *   draft_probs    [total_draft, vocab] fp32 q; request b's rows are
 *                  off[b] .. off[b] + gamma_b - 1.  Used as given (not
 *                  renormalised).  Only the gathered q(x_i) and the one residual
 *                  row per rejected request are read.  NULL selects a sparse q
 *                  (draft_topk > 0) or point-mass drafts (draft_topk == 0).
 *   draft_topk_ids / draft_topk_probs  [total_draft, draft_topk] int32 / fp32,
 *                  when draft_probs is NULL and draft_topk > 0: q of draft row d
 *                  is draft_topk_probs[d, s] at token draft_topk_ids[d, s] and 0
 *                  at every token not listed; id -1 marks an unused entry; the
 *                  ids of a row are distinct.  A residual draw then reads the
 *                  logits row and these entries only.
 *   draft_topk == 0 with draft_probs NULL: q_i is 1 at x_i and 0 elsewhere
 *                  (drafts proposed without a draft model); no q memory is read.
 *   draft_ids      [total_draft] int32 x_i, in [0, vocab).
 *   temperature    [batch] fp32; > 0 sampled, otherwise greedy.
 *   uniforms       [batch, gamma + 2] fp32 in [0, 1) (see the column map above).
 * Outputs (written for every request):
 *   out_tokens       [batch, gamma + 1] int32: drafts 0..k-1, then the drawn (or
 *                    greedy) token at k, then -1 (all -1 for a request that
 *                    breaks the device-side contract, see sv_device_error).
 *   out_num_accepted [batch] int32: k, the number of accepted drafts (-1 for
 *                    a request that breaks the contract).
 * Optional diagnostics (NULL to skip):
 *   diag_row_max   [total_draft + batch] fp32: max raw logit of every target row.
 *   diag_row_norm  [total_draft + batch] fp64: Z = sum exp((l - max) / T) of every
 *                  sampled row (0 for greedy rows).
 *   diag_ratio     [total_draft] fp32: p(x_i) / max(q(x_i), 1e-10) of every draft
 *                  of a sampled request (NaN for greedy requests).
 */
typedef struct sv_args {
    int32_t batch;               /* 0 .. max_batch (0 is a no-op) */
    int32_t gamma;               /* padded draft width, 0 .. max_gamma */
    int32_t total_draft;         /* sum of gamma_b (= batch * gamma when draft_offsets is NULL) */
    int32_t vocab;               /* must equal the context's vocab */
    const int32_t *draft_offsets;   /* [batch + 1] or NULL */
    const void    *target_logits;
    const float   *draft_probs;
    const int32_t *draft_ids;
    const float   *temperature;
    const float   *uniforms;
    int32_t *out_tokens;
    int32_t *out_num_accepted;
    float   *diag_row_max;
    double  *diag_row_norm;
    float   *diag_ratio;
    int32_t  draft_topk;            /* entries per sparse q row, 0 .. SV_MAX_TOPK (see above) */
    const int32_t *draft_topk_ids;  /* [total_draft, draft_topk] or NULL */
    const float   *draft_topk_probs;/* [total_draft, draft_topk] or NULL */
    uint32_t *stats;                /* [SV_STATS_LEN(gamma)] acceptance counters, or NULL */
} sv_args;

typedef struct sv_ctx sv_ctx;    /* opaque; owns the device scratch of one stream */

/* Creates a context for the verify step of the spec-decoding page (section 3.1:
 * B requests, gamma_b drafts each, gamma_b + 1 target distributions over one
 * vocabulary shared by draft and target, section 8 pitfall 1) on HIP device
 * `device`, and allocates what every call reuses: device scratch for the row
 * statistics, draw records and arrival counters sized for cfg's limits, a
 * pinned host word for contract violations (and one for reading it back) and
 * an internal non-blocking stream (with SV_FLAG_PROFILE also a ring of
 * events).  On success *out holds the context (free it with
 * spec_verify_destroy).  Returns SV_ERR_INVALID_ARG for bad limits,
 * SV_ERR_UNSUPPORTED for a dtype, vocab or row count (max_batch *
 * (max_gamma + 1) above 2^31 - 1) the library does not handle,
 * SV_ERR_OUT_OF_MEMORY / SV_ERR_DEVICE on HIP failure (then *out is NULL). */
int spec_verify_create(const sv_config *cfg, int device, sv_ctx **out);

/* Enqueues one verify step on `stream` (a hipStream_t; NULL = default stream)
 * and returns without waiting.  First, if the device has reported a contract
 * violation of an earlier call, returns SV_ERR_DEVICE_CONTRACT; then the
 * host-visible arguments are checked; on a non-SV_OK status nothing is
 * enqueued.  Outputs are valid once the stream has reached this point.  The
 * call allocates nothing.  One context must not be used by two streams at the
 * same time (its scratch is per call).  Without SV_FLAG_PROFILE the call only
 * launches kernels whose arrival counters reset themselves, so it may be
 * captured in a HIP graph and replayed (the buffers' contents may change
 * between replays; their addresses and the sizes may not). */
int spec_verify_run(sv_ctx *ctx, const sv_args *args, void *stream);

/* Releases what spec_verify_create allocated (lifecycle only; the page defines
 * no such step).  Waits for the stream of the context's last eagerly launched
 * call (it must still exist) and for the context's internal stream first, not
 * for other streams (freeing device memory may itself synchronise the device).
 * NULL is a no-op. */
int spec_verify_destroy(sv_ctx *ctx);

/* Reads (and, if clear != 0, resets) the sticky SV_DEVERR_* word.  Synchronises
 * the stream of the context's last eagerly launched call (it must still exist;
 * synchronise a replayed graph yourself) and uses the context's internal stream
 * for the read and the reset, so other streams are not waited for.  Do not call
 * it while a call on this context may still be enqueued elsewhere. */
int spec_verify_device_errors(sv_ctx *ctx, uint32_t *bits, int clear);

/* With SV_FLAG_PROFILE: waits for the recorded events and returns the summed
 * durations (milliseconds) over `*count` calls since the last read, then resets
 * the sums.  rows_ms is the row-statistics kernel and draw_ms the draw kernel,
 * each stamped by its own dispatch (start to end of the kernel's execution, the
 * gap between dispatches excluded). */
int spec_verify_profile_read(sv_ctx *ctx, double *rows_ms, double *draw_ms, int32_t *count);

/* Schedule the last successful spec_verify_run on this context launched. */
enum sv_schedule {
    SV_SCHEDULE_NONE = 0,       /* no call yet, or the last call had batch == 0 */
    SV_SCHEDULE_SPLIT = 1,      /* rows kernel with per-row pieces (unaligned rows), draw kernel */
    SV_SCHEDULE_FLAT = 2        /* rows kernel over the flattened rows, draw kernel */
};

/* Writes the sv_schedule of the last successful run to *schedule.  Host-only
 * (no device work); SV_ERR_INVALID_ARG on null pointers. */
int spec_verify_last_schedule(const sv_ctx *ctx, int32_t *schedule);

/* Static, human-readable name of a status code. */
const char *spec_verify_status_string(int status);

/* Limits of spec_verify_run_static. */
#define SV_STATIC_MAX_BATCH 256          /* requests per call */
#define SV_STATIC_MAX_ROWS 4096          /* target rows per call (total_draft + batch) */
#define SV_STATIC_MAX_DRAW_BLOCKS 32768  /* batch * ceil(vocab / 2048) per call */
#define SV_STATIC_SCRATCH_BYTES (8u << 20) /* device scratch per GPU, held until the process ends */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * verify step as spec_verify_run, with no context.  Its kernels use a
 * file-scope device array of SV_STATIC_SCRATCH_BYTES (one per GPU, set up on
 * the first call on that device, which must be the current device; no
 * hipMalloc, hipFree or allocating routine is ever called).  logits_dtype is
 * SV_F32 or SV_BF16; args->vocab may be any size up to 524288.  Returns
 * SV_ERR_CAPACITY for batch > SV_STATIC_MAX_BATCH, gamma > SV_MAX_GAMMA, more
 * than SV_STATIC_MAX_ROWS target rows or batch * ceil(vocab / 2048) above
 * SV_STATIC_MAX_DRAW_BLOCKS (128 requests at the largest vocab), else the
 * statuses of spec_verify_run
 * (nothing is enqueued unless SV_OK).  Every call on one GPU shares that GPU's
 * array and leaves it ready for the next: calls that overlap on one GPU (two
 * streams, or two threads) race and must be serialised by the caller.  A
 * request that breaks the device-side contract gets -1 outputs as with
 * spec_verify_run; no error word is reported. */
int spec_verify_run_static(int logits_dtype, const sv_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
