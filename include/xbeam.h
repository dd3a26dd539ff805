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

/* ---------------------------------------------------------------------------
 * Valid-path constraint (xGR summary, section 2.2, xBeam: beams may only
 * extend along token paths of a pre-built vocabulary of valid items; masks of
 * the early decode steps, which have many candidates, are stored densely and
 * pre-generated, those of later steps sparsely).
 *
 * The items form a trie.  The nodes at depth d are the distinct item
 * prefixes of length d, numbered 0.. in lexicographic order; the root is node
 * 0 of depth 0.  A beam that has generated d tokens of a valid path sits on
 * the node of that prefix; -1 marks a beam that has left every valid path.
 */

#define XATTN_TRIE_MAX_LEVELS 8

/* Layout of the tables inside one buffer; offsets are bytes from its start,
 * every section 256-byte aligned.  For depth d < levels:
 *   row_ptr   int32 [nodes[d] + 1]   edges of node n: row_ptr[n] .. row_ptr[n+1]-1
 *   child_tok int32 [nodes[d + 1]]   each edge's token, ascending within a node;
 *                                    edge e leads to node e of depth d + 1
 *   mask      uint32 [nodes[d]][words], only for d < dense_levels: bit j % 32
 *             of word j / 32 is set iff token j follows node n */
typedef struct {
  int32_t vocab;          /* tokens are 0 .. vocab-1 at every depth */
  int32_t levels;         /* tokens per item, L */
  int32_t dense_levels;   /* depths 0 .. dense_levels-1 carry dense masks */
  int32_t words;          /* (vocab + 31) / 32 */
  int32_t nodes[XATTN_TRIE_MAX_LEVELS + 1];
  int64_t row_ptr_off[XATTN_TRIE_MAX_LEVELS];
  int64_t child_tok_off[XATTN_TRIE_MAX_LEVELS];
  int64_t mask_off[XATTN_TRIE_MAX_LEVELS];
  int64_t total_bytes;
} xattn_trie;

/*
 * Host function, no device work: lays out the tables for n_items valid items
 * (items: HOST array [n_items][levels] int32, tokens in [0, vocab), any order,
 * duplicates allowed) and, when host_table is not NULL, fills host_table
 * (host memory of host_bytes >= layout->total_bytes).  Call once with
 * host_table = NULL for the size, then again to fill; copy the buffer to
 * device memory (any 256-byte-aligned address) for the kernels below.
 * 1 <= levels <= 8, 1 <= vocab <= 65536, 0 <= dense_levels <= levels,
 * 0 <= n_items < 2^31.
 */
xattn_status xattn_trie_build(const int32_t *items, int64_t n_items, int32_t levels,
                              int32_t vocab, int32_t dense_levels, xattn_trie *layout,
                              void *host_table, size_t host_bytes);

/*
 * Masks one decode step's logits in place: for every row (r, b), every token
 * that does not extend node[r * BW + b] (a node at `depth`) along a valid
 * path is set to -inf; valid tokens are left untouched (not rewritten).  A
 * dead beam (-1, or any id outside the depth's node range) gets a row of
 * -inf.
 *   layout, table   from xattn_trie_build; table is the DEVICE copy
 *   depth           0 <= depth < levels: tokens already generated
 *   node            [R][BW] int32, device
 *   logits          R * BW rows of vocab floats, device, 16-byte aligned, row
 *                   stride row_stride (elements, >= vocab, a multiple of 4)
 * The _timed form binds two caller events to the kernel dispatch.
 */
xattn_status xattn_valid_mask(const xattn_trie *layout, const void *table, int32_t depth,
                              const int32_t *node, float *logits, int32_t R, int32_t BW,
                              int64_t row_stride, void *stream);
xattn_status xattn_valid_mask_timed(const xattn_trie *layout, const void *table, int32_t depth,
                                    const int32_t *node, float *logits, int32_t R, int32_t BW,
                                    int64_t row_stride, void *stream, void *start_event,
                                    void *stop_event);

/*
 * Moves the beams one level down after selection: new beam b of request r
 * descends from slot parent[r * parent_stride + b] (clamped to [0, BW)) through
 * token[r * token_stride + b]; new_node[r * BW + b] is the child of
 * node[r * BW + parent] for that token at depth + 1, or -1 when the token
 * leaves the vocabulary (or the parent was dead).  parent and token can be the
 * outputs of xattn_beam_topk.  new_node must not overlap node.
 *   0 <= depth < levels; parent_stride, token_stride >= BW; all device arrays.
 */
xattn_status xattn_trie_advance(const xattn_trie *layout, const void *table, int32_t depth,
                                const int32_t *node, const int32_t *parent,
                                int64_t parent_stride, const int32_t *token,
                                int64_t token_stride, int32_t *new_node, int32_t R, int32_t BW,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* XBEAM_H */
