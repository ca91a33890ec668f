/*
 * moe_accept.h -- C ABI of greedy MTP verify/accept for AMD Instinct MI355X
 * (gfx950), the step that consumes the target's verify batch.
 *
 * "Support Step3.5/3.7 flash mtp3" (Overview, data-flow trace of one MTP
 * step, steps 4 "verify" and 5 "accept"): the target decodes the batch
 * [id_last, draft_1, ..., draft_{M-1}] with logits on for every row, so row
 * j's logits give the target's own token after batch token j.  Drafts are
 * kept while the target's token of row j equals draft_{j+1}; the first row
 * that disagrees supplies the token that replaces that draft, and if every
 * draft agrees the last row supplies one more token.  n_accepted counts the
 * agreeing drafts, the accepted list is those drafts followed by that one
 * token, and the hidden state carried into the next round is verify row
 * n_accepted (pending_h = verify_h[n_accepted]).
 *
 * Greedy sampling: the token of a row is the index of its largest logit,
 * the lower index where several are equal (the pages state no tie rule;
 * this is the library's).  Comparisons are exact on the fp32 values; -0 and
 * +0 compare equal; NaN counts as lower than every other value (the pages'
 * logits are finite, so this only fixes the behaviour for bad input).
 *
 * Status codes are those of moe_layer.h (MOE_OK, MOE_ERR_*).
 */
#ifndef SVR_MOE_ACCEPT_H
#define SVR_MOE_ACCEPT_H

#include <stddef.h>
#include <stdint.h>

#include "moe_layer.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest verify batch (rows) and vocabulary a call takes. */
#define MOE_ACCEPT_MAX_ROWS 64
#define MOE_ACCEPT_MAX_VOCAB 1073741824 /* 2^30 columns */

/* Device workspace, in *bytes, that moe_verify_accept needs for up to
 * max_rows rows of `vocab` columns: one 256-byte counter line, then one
 * 8-byte partial result per (workgroup, row).  The counter line must be
 * zero before the first call that uses the workspace; every call leaves it
 * zero again, so zero-fill a workspace once when it is allocated.  Calls
 * that share a workspace must not overlap in time.
 * MOE_ERR_NULL if bytes is NULL; MOE_ERR_SHAPE unless
 * 1 <= max_rows <= MOE_ACCEPT_MAX_ROWS and 1 <= vocab <= MOE_ACCEPT_MAX_VOCAB. */
int32_t moe_accept_workspace_bytes(int32_t max_rows, int64_t vocab, size_t* bytes);

/* Greedy verify/accept of one verify batch of M = n_rows rows, as ONE kernel
 * launch on hip_stream.  All pointers are DEVICE pointers owned by the
 * caller; nothing is allocated and the call returns without synchronising.
 *   logits     [M][vocab] float, row-major, read-only (any 4-byte alignment;
 *              16-byte aligned rows are read with 16-byte loads).
 *   drafts     [M-1] int32: draft_{j+1} at index j (may be NULL when M == 1).
 *   verify_h   [M][h_dim] float, the target's hidden state of each verify
 *              row; may be NULL, and then h_dim must be 0.
 *   tokens     [M] int32 out: the greedy token of every row.
 *   accepted   [M] int32 out: accepted[0..n_accepted] = the agreeing drafts
 *              followed by the target's token of row n_accepted; the
 *              entries after it are -1.
 *   n_accepted [1] int32 out.
 *   pending_h  [h_dim] float out: row n_accepted of verify_h (not written
 *              when verify_h is NULL).
 *   workspace  moe_accept_workspace_bytes(M, vocab) bytes, 256-byte
 *              aligned, counter line zero (see above).
 * Outputs must not alias inputs, each other or the workspace.
 * Errors (nothing enqueued): MOE_ERR_NULL for a NULL logits, tokens,
 * accepted, n_accepted or workspace pointer, for drafts NULL with M > 1, or
 * for exactly one of verify_h and pending_h NULL; MOE_ERR_SHAPE for M or
 * vocab out of range or h_dim < 0 (or h_dim > 0 without verify_h);
 * MOE_ERR_WORKSPACE for too small a workspace; MOE_ERR_ARG for a workspace
 * that is not 256-byte aligned or logits not 4-byte aligned; MOE_ERR_LAUNCH
 * if the launch fails.  n_rows == 0 enqueues nothing and returns MOE_OK
 * (after the shape checks). */
int32_t moe_verify_accept(const float* logits, int32_t n_rows, int64_t vocab,
                          const int32_t* drafts, const float* verify_h, int32_t h_dim,
                          int32_t* tokens, int32_t* accepted, int32_t* n_accepted,
                          float* pending_h, void* workspace, size_t workspace_bytes,
                          void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SVR_MOE_ACCEPT_H */
