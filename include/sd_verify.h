/*
 * sd_verify.h -- C ABI of the MI355X speculative-decoding verifier.
 *
 * The operation (pages cited by title and section):
 *   For every request b with k drafted tokens x[b,0..k-1] the target model's
 *   logits hold k+1 rows: one per draft position plus the bonus position
 *   (pyshine "vLLM, part 2", "Verification: rejection sampling on the GPU").
 *   Each row is masked by the grammar bitmask (same page, "Grammar gates":
 *   one mask row per request and per speculative position; forbidden tokens
 *   get probability zero), divided by the request's temperature, optionally
 *   truncated to its top-k tokens, and normalised over the vocabulary.
 *   Draft x_i is accepted with probability min(1, p_i(x_i) / q_i(x_i))
 *   (vllm-learning code walkthrough, RejectionSampler); without draft
 *   probabilities q is one-hot, so the acceptance probability is p_i(x_i)
 *   (infra-guide 5.2, section 4.3).  The scan stops at the first rejection,
 *   which is resampled from max(p - q, 0) renormalised; after full acceptance
 *   the bonus token is sampled from p_k; temperature 0 selects the greedy
 *   rule (accept while the draft equals the argmax, emit the argmax).  The
 *   call also emits the R/I/D/A counters (fanout, "Structured output
 *   speculative decoding acceptance", "Name the three counters").
 *
 *   Every uniform comes from Philox4x32-10 (Salmon et al., SC'11) keyed by
 *   the 64-bit seed: counter (0, i, b, 0) word 0 for the accept draw of
 *   position i of request b; (c >> 2, a, b, 1) word c & 3 for block c and
 *   (j >> 2, a, b, 2) word j & 3 for token j when row a is sampled.
 *   Sampling is two-level Gumbel-max over blocks of 2048 tokens.  Lowest
 *   index wins every tie.
 *
 * Conventions for every entry point:
 *   - "device" pointers address HIP device memory of the current device;
 *     "host" pointers address ordinary host memory.
 *   - Row-major layouts; the caller owns every buffer.  The library keeps no
 *     pointer after a call returns and allocates no device memory per call.
 *   - Calls are asynchronous on `stream`; calls on different streams with
 *     different workspaces may run concurrently.  No global RNG state exists.
 *   - The return value reports what the host can check (sd_status); data
 *     errors found on the device are reported through params->status.
 */
#ifndef SD_VERIFY_H
#define SD_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SD_OK = 0,
    SD_ERR_INVALID_ARG = -1, /* null required pointer, negative size, bad dtype */
    SD_ERR_UNSUPPORTED = -2, /* B > SD_MAX_BATCH, k > SD_MAX_DRAFT or V > SD_MAX_VOCAB */
    SD_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    SD_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
    SD_ERR_SCRATCH_LIMIT = -5 /* sd_verify_noalloc: the call needs more than
                                 SD_NOALLOC_SCRATCH_BYTES of workspace */
} sd_status;

typedef enum { SD_DTYPE_F32 = 0, SD_DTYPE_BF16 = 1 } sd_dtype;

#define SD_MAX_BATCH 65535        /* largest supported B per call */
#define SD_MAX_DRAFT 64           /* largest supported k */
#define SD_MAX_VOCAB (1 << 22)    /* largest supported V (2048 blocks of 2048) */
#define SD_BLOCK_TOKENS 2048      /* level-1 block of the two-level Gumbel-max */

/* Data-error bits OR-ed into *params->status.  A request with any bit set
 * gets out_tokens = -1 in every slot, out_num_accepted = -1, and adds nothing
 * to the counters. */
#define SD_STATUS_DRAFT_ID 1u       /* a draft id outside [0, V) */
#define SD_STATUS_TEMPERATURE 2u    /* temperature negative, NaN or infinite */
#define SD_STATUS_EMPTY_ROW 4u      /* a row without an allowed finite logit */
#define SD_STATUS_BAD_LOGIT 8u      /* NaN or +inf logit at an allowed token */
#define SD_STATUS_BAD_DRAFT_PROB 16u /* q at a draft token NaN, infinite or < 0 */
#define SD_STATUS_BAD_OFFSETS 32u   /* ragged call whose draft offsets are inconsistent:
                                       set on every request (see draft_offsets) */

/* Debug-only timing hooks, not part of the verification contract (callers
 * that only verify leave the pointer to them NULL): hipEvent_t handles that a
 * call records on its stream immediately before and after its main kernel
 * (the sweep for sd_verify, the match kernel for sd_ngram_propose), so that a
 * benchmark can time that kernel alone.  A NULL handle is skipped. */
typedef struct {
    void *kernel_begin;
    void *kernel_end;
} sd_debug_timing;

typedef struct {
    int32_t batch;      /* B, 0 <= B <= SD_MAX_BATCH requests */
    int32_t num_draft;  /* k, 0 <= k <= SD_MAX_DRAFT, the same for every request */
    int32_t vocab;      /* V, 1 <= V <= SD_MAX_VOCAB */
    sd_dtype logits_dtype;
    /* device [B] or NULL: top-k per request, <= 0 = off.  A sampling request
     * keeps every allowed token whose logit is >= its top_k-th largest allowed
     * logit (ties kept), at every position (pyshine, "Verification": top-k
     * applied with temperature before the accept test).  Greedy ignores it. */
    const int32_t *top_k;
    /* Optional device outputs for parity checks (NULL = not written):
     *   dbg_row_lse     [B, k+1]  log sum exp(l/T) over each row's support
     *                             (greedy rows: the largest allowed logit)
     *   dbg_accept_prob [B, k]    min(1, p/q) (greedy: 1 if x == argmax else 0)
     *   dbg_request_flags [B]     per request: boundary accept draws
     *                             (|u - a| < 1e-6) in bits 0..11, Gumbel near
     *                             ties (top-2 keys closer than 1e-5) in bits
     *                             12..23, top-p boundary rows (the mass at
     *                             the cut, or just above it, within 1e-9 of
     *                             top_p, relative to the row's kept mass) in
     *                             bits 24..31
     *   dbg_flags [3]             totals of the three flag kinds over the call */
    double *dbg_row_lse;
    double *dbg_accept_prob;
    uint32_t *dbg_request_flags;
    uint32_t *dbg_flags;
    /* device [1] or NULL: OR of the SD_STATUS_* bits of all requests
     * (overwritten by every call). */
    uint32_t *status;
    /* Debug only, NULL in production: timing hooks (sd_debug_timing). */
    const sd_debug_timing *debug_timing;
    /* Ragged draft lengths (infra-guide 5.2, drafters that propose a variable
     * number of tokens), or NULL for k drafts per request.  device [B + 1]
     * int32 cumulative offsets: request b verifies k_b = off[b+1] - off[b]
     * drafts, 0 <= k_b <= num_draft.  Every per-row and per-draft array is
     * then packed without padding: logits and bitmask [total_drafts + B, ...]
     * with request b's k_b + 1 rows from row off[b] + b, draft_token_ids
     * [total_drafts] and draft_probs [total_drafts, V] from draft off[b],
     * out_tokens [total_drafts + B] (k_b + 1 slots from off[b] + b),
     * dbg_row_lse [total_drafts + B], dbg_accept_prob [total_drafts].  The
     * offsets must start at 0, never decrease and end at total_drafts;
     * otherwise every request gets SD_STATUS_BAD_OFFSETS and
     * out_num_accepted = -1, no out_tokens slot is written and the counters
     * are 0. */
    const int32_t *draft_offsets;
    int64_t total_drafts;  /* host: off[B] of a ragged call, 0 <= total_drafts <= B * num_draft */
    /* device [num_draft + 1] or NULL: requests per accepted draft length
     * (fanout, "Mean acceptance length uses another denominator": one bucket
     * per possible accepted length), requests in error left out; overwritten
     * by every call.  Accepted drafts per position i follow as the sum of
     * the buckets above i. */
    uint32_t *accept_histogram;
    /* device [B] or NULL: top-p per request, applied after top-k; values
     * outside (0, 1) switch it off.  A sampling request keeps, at every row,
     * the allowed tokens whose logit is >= the largest value v such that the
     * tokens >= v hold top_p of the tempered mass left by top-k (ties at v
     * kept).  Greedy ignores it. */
    const float *top_p;
} sd_params;

/* Bytes of device workspace sd_verify needs for these sizes (0 for B = 0),
 * including total_drafts for a ragged call, and a table of line maxima when
 * top_k is not NULL (any non-NULL value: calls that pass top_k need this
 * larger size).  Host-only; never fails (returns 0 for invalid sizes). */
size_t sd_verify_workspace_size(const sd_params *p);

/* Verify one batch (shapes below for k drafts per request; see
 * sd_params.draft_offsets for ragged calls).
 *   target_logits     device [B, k+1, V] bf16 or fp32 (p->logits_dtype).
 *                     Rows 16-byte aligned take the vector path, others a
 *                     slower element path.
 *   draft_token_ids   device [B, k] int32 (may be NULL when k = 0)
 *   draft_probs       device [B, k, V] fp32, or NULL for one-hot drafts
 *   bitmask           device [B, k+1, ceil(V/32)] int32, bit (j & 31) of word
 *                     j >> 5 set = token j allowed (bits >= V ignored), or NULL
 *   temperature       device [B] fp32; 0 = greedy
 *   seed              Philox key
 *   out_tokens        device [B, k+1] int32: accepted drafts, then the
 *                     resampled/bonus/argmax token, then -1
 *   out_num_accepted  device [B] int32
 *   out_counters      device [4] uint64 = R, I, D, A of this call (overwritten)
 *   p                 host pointer to the sizes and optional outputs
 *   workspace         device scratch of >= sd_verify_workspace_size(p) bytes,
 *                     256-byte aligned, zero-filled once before its first
 *                     use (hipMemset): its first 16 KB hold the row sweep's
 *                     block-claim counters, which every call that launches
 *                     returns to zero, so a workspace stays ready for calls
 *                     of any size; the rest is scratch.  After a call that
 *                     returned SD_ERR_HIP, zero it again.  Must not be shared
 *                     by calls that overlap in time
 * Returns SD_OK or a negative sd_status; nothing is launched on error. */
int sd_verify(const void *target_logits, const int32_t *draft_token_ids,
              const float *draft_probs, const int32_t *bitmask,
              const float *temperature, uint64_t seed, int32_t *out_tokens,
              int32_t *out_num_accepted, uint64_t *out_counters,
              const sd_params *p, void *workspace, size_t workspace_bytes,
              hipStream_t stream);

/* Bytes of the static device scratch behind sd_verify_noalloc: every call
 * whose sd_verify_workspace_size is at most this fits (the B=512, k=12,
 * V=151936 long-draft shape with top-k needs about 42 MB). */
#define SD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* sd_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same operation, arguments and outputs as sd_verify, without the workspace
 * arguments: the workspace is a static device array of
 * SD_NOALLOC_SCRATCH_BYTES, one per device, held from the first call on that
 * device until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); the caller still owns every input and
 * output buffer.
 *   - The first call on a device looks the array up with
 *     hipGetSymbolAddress and clears its block-claim counters with a fill
 *     kernel on `stream`; every later call finds them at zero, since every
 *     call that launches leaves them so (after an SD_ERR_HIP the next call
 *     clears them again).
 *   - Every call on one device shares that device's array: calls that
 *     overlap in time on one device (different streams or threads) race and
 *     produce garbage.  Serialise them.
 * Returns what sd_verify returns, SD_ERR_SCRATCH_LIMIT when
 * sd_verify_workspace_size(p) exceeds SD_NOALLOC_SCRATCH_BYTES, and
 * SD_ERR_HIP when the array cannot be looked up; nothing is launched on
 * error. */
int sd_verify_noalloc(const void *target_logits, const int32_t *draft_token_ids,
                      const float *draft_probs, const int32_t *bitmask,
                      const float *temperature, uint64_t seed, int32_t *out_tokens,
                      int32_t *out_num_accepted, uint64_t *out_counters,
                      const sd_params *p, hipStream_t stream);

/* Static description of a return code.  Host-only. */
const char *sd_status_string(int code);

/* Ratios over the counters (fanout, "Name the three counters" and "Mean
 * acceptance length uses another denominator"): survival D/R, acceptance
 * A/D, yield A/R, mean acceptance length 1 + A/steps.  A ratio whose
 * denominator is zero is written as NaN.  counters: host [4] = R, I, D, A;
 * out: host [4].  Returns SD_ERR_INVALID_ARG for NULL pointers or counters
 * with D != R - I or A > D.  Host-only. */
int sd_rates(const uint64_t *counters, uint64_t steps, double *out);

#ifdef __cplusplus
}
#endif

#endif /* SD_VERIFY_H */
