/*
 * xbeam.h -- beam selection in libxattn.so: the step that follows attention
 * in beam-search generative recommendation and produces the parent slots
 * the next step's attention reads (parent_idx in xattn.h).
 *
 * The operation is the top-K of the xBeam component of the xGR technical
 * summary (gist.science, paper 2512.11529), section 2.2, over the candidate
 * pools of its section 1 (128 x 128 and 512 x 512): every live beam proposes
 * its candidates sorted by log-probability, a candidate's score is the
 * beam's cumulative score plus its log-probability, and the BW best of all
 * BW x V candidates become the next step's beams.  The page finds them with
 * a min-heap and stops scanning a beam's sorted list once the next
 * candidate cannot enter; the kernel here keeps that early termination
 * (sorted rows cut every row's scan at a threshold) in a form a workgroup
 * runs in parallel.
 *
 * Definitions fixed here where the page is silent:
 *   - score(b, j) = cum[b] + logp[b][j], one IEEE float32 addition rounded to
 *     nearest even;
 *   - order: score descending, then parent beam ascending, then token id
 *     ascending (signed int32 order); the selection is unique under it;
 *   - output i (0 <= i < BW) is the i-th best candidate in that order.
 *
 * Conventions are those of xattn.h: device pointers to caller-owned dense
 * row-major memory, asynchronous on `stream`, status codes with a reason in
 * xattn_last_error(), every host-checkable argument checked before anything
 * is enqueued.
 */
#ifndef XBEAM_H
#define XBEAM_H

#include <stdint.h>

#include "xattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest beam width xattn_beam_topk takes. */
#define XBEAM_MAX_BEAMS 512

/*
 * The BW best next beams of each of R requests.
 *
 *   cum        [R][BW] float32        cumulative score of every live beam
 *   logp       [R][BW][V] float32     each beam's candidate log-probabilities,
 *                                     every row non-increasing (the kernel's
 *                                     early termination relies on it)
 *   token      [R][BW][V] int32       the token id of each candidate
 *   R >= 1, 1 <= BW <= XBEAM_MAX_BEAMS, 1 <= V <= 2^24
 *   new_score  written: new_score[r * out_stride + i], i < BW, the score of
 *              the i-th best candidate of request r
 *   new_parent written likewise: the beam (0..BW-1) it extends; with
 *              out_stride = S * BW this writes row t of a parent_idx
 *              [R][S][BW] array directly (pass parent_idx + t * BW)
 *   new_token  written likewise: its token id
 *   out_stride >= BW, elements between consecutive requests' outputs
 *
 * All arrays 4-byte aligned; outputs must not overlap inputs or each other.
 * Values are preconditions, not checked: no NaN score (cum + logp must not
 * be NaN; -inf marks a masked candidate and is allowed) and sorted rows.  A
 * violation gives unspecified output but no out-of-bounds access.
 */
xattn_status xattn_beam_topk(const float *cum, const float *logp, const int32_t *token,
                             int32_t R, int32_t BW, int32_t V, float *new_score,
                             int32_t *new_parent, int32_t *new_token, int64_t out_stride,
                             void *stream);

/*
 * xattn_beam_topk for measurement: the same work and results; start_event
 * and stop_event (hipEvent_t, both required) are bound to the kernel's own
 * dispatch, as in xattn_decode_timed.
 */
xattn_status xattn_beam_topk_timed(const float *cum, const float *logp, const int32_t *token,
                                   int32_t R, int32_t BW, int32_t V, float *new_score,
                                   int32_t *new_parent, int32_t *new_token, int64_t out_stride,
                                   void *stream, void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* XBEAM_H */
