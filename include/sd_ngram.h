/*
 * sd_ngram.h -- C ABI of the MI355X n-gram (prompt lookup) draft proposer.
 *
 * The operation (pages cited by title and section):
 *   For each request the last n tokens of its history (prompt and generated
 *   tokens alike, compared by id) are looked up earlier in the same history
 *   and the tokens that followed that earlier occurrence are proposed as
 *   drafts (infra-guide 5.2 "Draft models and model-free methods", section
 *   4.1 "Match the tail, then copy what follows").  The window n runs from
 *   max_n, never more than len - 1, down to min_n and the longest window that
 *   occurs wins; among its occurrences the one that starts earliest wins; an
 *   occurrence may overlap the tail but is never the tail itself (same page,
 *   section 6 "Hands-on: match window and candidate coverage"; pyshine "vLLM,
 *   part 2", "Choosing a drafter").  Up to k tokens are copied, fewer when
 *   the history ends first.  A history with no occurrence, one too short for
 *   min_n, or one whose k drafts would run past the model's context length
 *   (len + k > max_model_len) gets no drafts (pyshine, "Choosing a drafter").
 *
 * The drafts come out both padded ([B, k], -1 after each request's drafts)
 * and, on request, in the ragged layout sd_verify takes: cumulative draft
 * offsets [B + 1] and the drafts back to back.
 *
 * Conventions are those of sd_verify.h: device pointers address HIP device
 * memory of the current device, layouts are row-major, the caller owns every
 * buffer, nothing is allocated per call, calls are asynchronous on `stream`,
 * and the return value is an sd_status.
 */
#ifndef SD_NGRAM_H
#define SD_NGRAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "sd_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SD_NGRAM_MAX_N 256        /* largest supported max_n */
#define SD_NGRAM_MAX_BATCH 65535  /* largest supported B per call */

/* Data-error bit written to *params->status (the OR over the batch; the
 * word is overwritten by every call). */
#define SD_NGRAM_STATUS_BAD_LENGTH 1u /* lengths[b] outside [0, stride]: no drafts for b */

typedef struct {
    int32_t batch;          /* B, 0 <= B <= SD_NGRAM_MAX_BATCH */
    int32_t min_n;          /* shortest window, 1 <= min_n */
    int32_t max_n;          /* longest window, min_n <= max_n <= SD_NGRAM_MAX_N */
    int32_t num_draft;      /* k, 0 <= k <= SD_MAX_DRAFT: most tokens proposed per request */
    int64_t stride;         /* tokens between rows of the history table, 1 <= stride < 2^31 */
    int64_t max_model_len;  /* context length: len + k above it gets no drafts; 0 = no limit */
    /* optional outputs (NULL = not written) */
    int32_t *out_match_len;     /* device [B]: the winning window n, 0 = no drafts */
    int32_t *out_draft_offsets; /* device [B + 1]: cumulative draft counts, offsets[0] = 0 */
    int32_t *out_drafts_flat;   /* device [B * k]: the drafts back to back, in the order
                                   of out_draft_offsets (needs out_draft_offsets); slots
                                   past offsets[B] are left as they were */
    uint32_t *status;           /* device [1]: SD_NGRAM_STATUS_* bits of the call */
    /* debug only, NULL in production: timing hooks (sd_debug_timing, sd_verify.h) */
    const sd_debug_timing *debug_timing;
} sd_ngram_params;

/* Device workspace bytes sd_ngram_propose needs for these sizes (0 when the
 * sizes are unsupported or B = 0). */
size_t sd_ngram_workspace_size(const sd_ngram_params *p);

/* Proposes drafts for B requests.
 *   tokens          device [B, stride] int32: row b holds request b's history in
 *                   its first lengths[b] entries; the rest is never read
 *   lengths         device [B] int32: history lengths
 *   out_drafts      device [B, k] int32: request b's drafts, then -1
 *   out_num_drafts  device [B] int32: how many drafts request b got (0..k)
 *   workspace       device, 256-byte aligned, sd_ngram_workspace_size(p) bytes;
 *                   its contents need no initialisation and are scratch after
 *                   the call
 * A request whose length is outside [0, stride] gets no drafts and sets
 * SD_NGRAM_STATUS_BAD_LENGTH.  Returns SD_OK, SD_ERR_INVALID_ARG (NULL
 * pointer, window or size out of range, flat drafts without offsets),
 * SD_ERR_UNSUPPORTED (B, k or max_n above its limit), SD_ERR_WORKSPACE or
 * SD_ERR_HIP; nothing is launched on error. */
int sd_ngram_propose(const int32_t *tokens, const int32_t *lengths, int32_t *out_drafts,
                     int32_t *out_num_drafts, const sd_ngram_params *p, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SD_NGRAM_H */
