/*
 * xattn.h -- C ABI of libxattn.so: staged decode attention for beam-search
 * generative recommendation on AMD Instinct MI355X (gfx950).
 *
 * The operation is the xAttention operator of the xGR technical summary
 * (gist.science, paper 2512.11529), section 2.1:
 *   - the KV cache is split into a Shared part, holding the prompt (user
 *     history) K/V computed once at prefill and stored once per request, and
 *     an Unshared part holding only the K/V of tokens generated during
 *     decode, one row per (level, beam slot) with no block alignment;
 *   - when beams branch nothing is copied: a beam reaches its generated
 *     tokens through the per-step parent-slot indices;
 *   - attention runs in three stages: the Shared and Unshared stages each
 *     produce local scores with max/sum statistics, and a Merging stage
 *     combines them with OnlineSoftmax.
 * Because the merge is exact, for query head h of beam b in request r the
 * result equals softmax attention over the concatenated keys
 *     [ shared rows 0..L_r-1 of KV head k ; the beam's ancestor token at
 *       every level 0..step of KV head k ],   k = h / (Hq / Hkv),
 * scaled by `scale` (default 1/sqrt(D)).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers to caller-owned, dense,
 *     row-major memory with the strides implied by the shape; the library
 *     allocates nothing and keeps no state between calls.
 *   - q, K, V and out share one element type (xattn_dtype).  Their base
 *     pointers must be 16-byte aligned; int32 arrays 4-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  Inputs must stay unchanged, and outputs are valid, only once
 *     the stream has reached the enqueued work.
 *   - Errors are status codes.  Every argument the host can check is checked
 *     before anything is enqueued (XATTN_EINVAL / XATTN_EUNSUPPORTED); a HIP
 *     launch failure returns XATTN_EHIP.  Nothing aborts, throws or prints;
 *     xattn_last_error() gives a one-line reason for the calling thread.
 *   - Values that live in device memory are preconditions, not checked:
 *     0 <= prompt_len[r] <= max_prompt_len and 0 <= parent_idx < beam_width.
 *     A violation gives unspecified output but no out-of-bounds access: the
 *     kernels clamp both before forming addresses.
 *   - Calls that share no output buffer may run concurrently.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XATTN_OK = 0,
  XATTN_EINVAL = 1,        /* an argument violates the contract below */
  XATTN_EUNSUPPORTED = 2,  /* valid, but not a supported head_dim / dtype */
  XATTN_EHIP = 3           /* the HIP runtime reported an error */
} xattn_status;

typedef enum {
  XATTN_F32 = 0,   /* float32 inputs and output; fp32 arithmetic throughout */
  XATTN_BF16 = 1   /* bfloat16 inputs and output; fp32 accumulation, output
                      rounded to nearest even */
} xattn_dtype;

typedef struct {
  int32_t num_requests;    /* R  >= 1 */
  int32_t beam_width;      /* BW >= 1: beam slots per level */
  int32_t num_q_heads;     /* Hq >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;        /* D: 64 or 128 */
  int32_t max_prompt_len;  /* Lmax >= 0: row capacity of the shared cache */
  int32_t max_steps;       /* S >= 1: level capacity of the unshared cache */
  int32_t dtype;           /* an xattn_dtype */
  float scale;             /* softmax scale, finite and >= 0; 0 selects 1/sqrt(D) */
} xattn_shape;

/*
 * One decode step of staged attention (the operation described above).
 *
 *   q           [R][BW][Hq][D]        query of every beam and head at `step`
 *   shared_k/v  [R][Hkv][Lmax][D]     prompt K/V; rows < prompt_len[r] are read
 *   prompt_len  [R] int32             L_r
 *   unshared_k/v[R][Hkv][S][BW][D]    generated-token K/V, one row per (level,
 *                                     slot); levels 0..step are read, so the
 *                                     caller writes level `step` first
 *   parent_idx  [R][S][BW] int32      parent_idx[r][t][b] = slot at level t-1
 *                                     that the level-t beam in slot b extends;
 *                                     rows 1..step are read, row 0 never
 *   step        0 <= step < S         current level s
 *   out         [R][BW][Hq][D]        written, same dtype as q
 *   (Calls with at most 8 query rows per request and KV head -- BW * Hq / Hkv
 *   <= 8, i.e. one or two beams -- are run by the per-beam kernel described
 *   below: with so few rows there is nothing to share, and the result is the
 *   same within rounding.)
 *   workspace   device scratch of at least xattn_workspace_size(shape, step)
 *               bytes, 256-byte aligned; may be NULL when that size is 0.
 *               Its contents on entry are ignored; two calls in flight at
 *               once must not share one workspace.
 */
xattn_status xattn_decode(const xattn_shape *shape, const void *q, const void *shared_k,
                          const void *shared_v, const int32_t *prompt_len,
                          const void *unshared_k, const void *unshared_v,
                          const int32_t *parent_idx, int32_t step, void *out,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * xattn_decode that also reports the ancestor slots its Unshared stage
 * gathered (xGR summary, section 2.1: a beam reaches its generated tokens
 * through the parent indices, token by token, with no copies):
 *   anc [R][step+1][BW] int32, written: anc[r][t][b] = the slot of beam b's
 *       ancestor at level t, i.e. anc[r][step][b] = b and
 *       anc[r][t-1][b] = parent_idx[r][t][anc[r][t][b]] for t = step..1.
 * Every other argument, the result and the errors are xattn_decode's, and
 * the call enqueues exactly xattn_decode's kernels (xattn_plan_decode): the
 * slots come from the code that walks the chain on the decode path.  Chains
 * of at most 16 levels are walked inside the attention kernel, which writes
 * the slots it walked to `anc`; deeper chains are resolved by the walk
 * kernels into the workspace, from which they are copied to `anc` on the
 * same stream.  Returns XATTN_EINVAL if anc is NULL or not 4-byte aligned.
 */
xattn_status xattn_decode_with_ancestors(const xattn_shape *shape, const void *q,
                                         const void *shared_k, const void *shared_v,
                                         const int32_t *prompt_len, const void *unshared_k,
                                         const void *unshared_v, const int32_t *parent_idx,
                                         int32_t step, void *out, int32_t *anc, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * xattn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument.  Arguments, result and errors are otherwise
 * xattn_decode's, and the kernels are the same.  A step that needs a
 * workspace (chains of more than 16 levels) uses a scratch array of
 * XATTN_NOALLOC_SCRATCH_BYTES inside the library instead: one per GPU,
 * which that GPU holds from the library's first use on it until the process
 * ends.  The call allocates nothing.
 *   - A shape and step whose xattn_workspace_size exceeds
 *     XATTN_NOALLOC_SCRATCH_BYTES is rejected with XATTN_EINVAL before
 *     anything is enqueued.
 *   - The scratch is the current device's (hipGetDevice): `stream` must
 *     belong to it.
 *   - Every call on a GPU shares that GPU's scratch, and each call leaves
 *     its contents behind; no call needs them cleared (every byte a call
 *     reads it wrote first).  Calls that may overlap on one GPU -- on
 *     different streams, or from different threads -- race on it: order
 *     them on one stream, or use xattn_decode with a workspace per stream.
 */
#define XATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
xattn_status xattn_decode_noalloc(const xattn_shape *shape, const void *q, const void *shared_k,
                                  const void *shared_v, const int32_t *prompt_len,
                                  const void *unshared_k, const void *unshared_v,
                                  const int32_t *parent_idx, int32_t step, void *out,
                                  void *stream);

/* Bytes of device workspace xattn_decode / xattn_decode_debug need for this
 * shape and step (0 if none).  Returns (size_t)-1 if the shape or step is
 * invalid.  Chains of more than 16 levels need it: the resolved ancestor
 * slots, and for bf16 the Unshared stage's partial (m, l, o) of every query
 * row, which a first kernel computes with one workgroup per (request, beam,
 * KV head) before the attention kernel starts from them.  When such a bf16
 * call has fewer than 128 (request, KV head, row block) workgroups and
 * a prompt of at least 8 tiles of 64 keys, each workgroup's prompt tiles
 * are split over up to 4 workgroups; the workspace then also holds every
 * split's partial (m, l, o) per query row, which a last kernel merges. */
size_t xattn_workspace_size(const xattn_shape *shape, int32_t step);

/*
 * The ancestor slots a beam reaches through the parent chain (xGR summary,
 * section 2.1: generated tokens are kept per token and reached without
 * copies when beams branch), on their own:
 *   anc [R][BW][step+1] int32, written: anc[r][b][step] = b and
 *   anc[r][b][t-1] = parent_idx[r][t][anc[r][b][t]] for t = step..1.
 * Runs the chunked walk kernel that xattn_decode uses for chains of more
 * than 16 levels that fit one segment (xattn_plan.ancestor_walk == 1).
 * xattn_decode_with_ancestors reports the slots of the decode path itself,
 * whichever walk it takes.
 */
xattn_status xattn_resolve_ancestors(const xattn_shape *shape, const int32_t *parent_idx,
                                     int32_t step, int32_t *anc, void *stream);

/*
 * xattn_decode that also exposes the stages (xGR summary, section 2.1: the
 * Shared and Unshared stages each produce max/sum statistics, and the
 * Merging stage combines them).  In this variant the two stages are kept
 * apart and merged explicitly; out matches xattn_decode's to within
 * rounding.  The stages run the decode path's own code: the Shared stage
 * the same prompt-tile loop, and the Unshared stage the same gathered
 * token blocks on the matrix cores (chains of at most 16 levels) or the
 * same per-beam token kernel (deeper chains), folded into a state of its
 * own instead of the shared one.  Running maxima here are exact (the
 * decode path raises them lazily), and a deep chain's prompt is never
 * split over workgroups.  Every tap is optional (NULL skips it):
 *   lse       [R][BW][Hq] float32     m + ln(sum), the merged log-normaliser
 *   stage_ml  [2][R][BW][Hq][2] f32   (m, l) per stage: stage 0 Shared,
 *                                     stage 1 Unshared; m = max scaled score,
 *                                     l = sum exp(score - m).  An empty
 *                                     prompt gives m = -inf, l = 0.
 *   stage_o   [2][R][BW][Hq][D] f32   per-stage normalised output
 *                                     (0 for an empty prompt)
 */
xattn_status xattn_decode_debug(const xattn_shape *shape, const void *q, const void *shared_k,
                                const void *shared_v, const int32_t *prompt_len,
                                const void *unshared_k, const void *unshared_v,
                                const int32_t *parent_idx, int32_t step, void *out,
                                float *lse, float *stage_ml, float *stage_o, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * xattn_decode for measurement: identical work and results, and in addition
 * start_event / stop_event (hipEvent_t, created by the caller, both required)
 * are bound to the kernel dispatches of the call -- start to the first
 * kernel's, stop to the last one's -- so hipEventElapsedTime(start_event,
 * stop_event) is the call's execution time on the device, with no queue or
 * marker latency around it.  A call is one kernel, or for chains deeper than
 * 16 levels up to five (the ancestor slots in one or two kernels, the
 * Unshared stage for bf16, attention, and the merge of key splits when the
 * grid is small).  Binding the events costs the device a few microseconds per
 * call around the dispatch, so a caller measuring throughput times a sample
 * of its calls this way and issues the rest through xattn_decode.
 * Returns XATTN_EINVAL if an event is NULL.
 */
xattn_status xattn_decode_timed(const xattn_shape *shape, const void *q, const void *shared_k,
                                const void *shared_v, const int32_t *prompt_len,
                                const void *unshared_k, const void *unshared_v,
                                const int32_t *parent_idx, int32_t step, void *out,
                                void *workspace, size_t workspace_bytes, void *stream,
                                void *start_event, void *stop_event);

/*
 * The same attention computed per beam, as a per-sequence decode kernel
 * (PagedAttention style) would: every (request, beam, KV head) streams the
 * beam's whole sequence, prompt included, so the prompt's K/V are read once
 * per beam instead of once per request.  This is the baseline the xGR
 * summary compares xAttention against (sections 1 and 4); it is kept to
 * measure that comparison on this hardware.  Arguments, layouts, workspace
 * and errors as xattn_decode; out matches xattn_decode's within rounding.
 * For XATTN_F32 it runs the float32 kernel, which already works per query
 * row.  The _timed form binds two caller events to the kernel dispatch, as
 * xattn_decode_timed does.
 */
xattn_status xattn_decode_per_beam(const xattn_shape *shape, const void *q, const void *shared_k,
                                   const void *shared_v, const int32_t *prompt_len,
                                   const void *unshared_k, const void *unshared_v,
                                   const int32_t *parent_idx, int32_t step, void *out,
                                   void *workspace, size_t workspace_bytes, void *stream);
xattn_status xattn_decode_per_beam_timed(const xattn_shape *shape, const void *q,
                                         const void *shared_k, const void *shared_v,
                                         const int32_t *prompt_len, const void *unshared_k,
                                         const void *unshared_v, const int32_t *parent_idx,
                                         int32_t step, void *out, void *workspace,
                                         size_t workspace_bytes, void *stream, void *start_event,
                                         void *stop_event);

/*
 * In-place reorder of the Unshared cache after beam selection (xGR summary,
 * section 2.1: generated-token blocks are updated in place, with direct
 * indices, free of write-before-read hazards).  The alternative to following
 * parent chains: afterwards slot b holds beam b's own history, and the next
 * step's attention can use identity parents.
 *
 *   unshared_k/v [R][Hkv][S][BW][D]   updated in place: for every request r,
 *                                     KV head, level t < n_levels and slot b,
 *                                     row (t, b) takes the old row
 *                                     (t, parent[r * parent_stride + b])
 *   parent       [R] rows of BW int32, row stride parent_stride >= BW; pass
 *                parent_idx + s * BW with stride S * BW to use row s of a
 *                parent_idx [R][S][BW] array.  Values outside [0, BW) are
 *                clamped (a precondition, as for parent_idx).
 *   n_levels     0 <= n_levels <= S; levels >= n_levels are not touched
 *
 * Typical use after the selection that yields the parents of level s+1:
 * reorder levels 0..s with them, then write level s+1 of every slot.  Within
 * every slice (request, KV head, level), all reads of a column range finish
 * before any of its rows is written, so the result is as if all rows were
 * read before any was written.  shape supplies R, BW, Hkv, D, S and dtype (head counts and
 * max_prompt_len must be valid but are otherwise unused); beam_width up to
 * 2048 (XATTN_EUNSUPPORTED above).  Calls on one cache must not overlap
 * each other or an attention call reading it.  The _timed form binds two
 * caller events to the kernel dispatch, as xattn_decode_timed does.
 */
xattn_status xattn_reorder_unshared(const xattn_shape *shape, void *unshared_k, void *unshared_v,
                                    const int32_t *parent, int64_t parent_stride,
                                    int32_t n_levels, void *stream);
xattn_status xattn_reorder_unshared_timed(const xattn_shape *shape, void *unshared_k,
                                          void *unshared_v, const int32_t *parent,
                                          int64_t parent_stride, int32_t n_levels, void *stream,
                                          void *start_event, void *stop_event);

/*
 * Where each call's work goes: what xattn_decode enqueues for a shape and
 * step, computed on the host alone (no device is touched; usable without a
 * GPU).  xattn_decode follows exactly this plan.
 */
typedef enum {
  XATTN_KERNEL_STAGED_BF16 = 0,   /* bf16: the staged MFMA kernel, one workgroup per
                                     compute unit, two waves per 32 query rows (one
                                     per half of each 64-key tile) */
  XATTN_KERNEL_F32 = 1,           /* float32: one workgroup per query row */
  XATTN_KERNEL_PER_BEAM_BF16 = 2, /* bf16 with <= 8 query rows per request and KV head */
  XATTN_KERNEL_STAGED_BF16_PAIRED = 3 /* bf16, grids of >= 512 workgroups of 128 rows:
                                     the same stages with one wave per 32 query rows on
                                     32-key tiles, <= 80 KiB of LDS, two workgroups per
                                     compute unit */
} xattn_kernel;

typedef struct {
  int32_t kernel;            /* an xattn_kernel: the attention kernel */
  int32_t kernels;           /* kernels one call enqueues, 1 to 5 */
  int32_t ancestor_walk;     /* 0: inside the attention kernel (<= 16 levels);
                                1: one chunked walk kernel; 2: the segmented walk
                                (two kernels), both into the workspace */
  int32_t unshared_kernel;   /* 1: a per-beam kernel computes the Unshared stage
                                first (bf16 chains deeper than 16 levels) */
  int32_t key_splits;        /* 1, or the workgroups each prompt is split over,
                                whose partials a last kernel merges */
  int32_t rows_per_block;    /* query rows per attention workgroup */
  int32_t threads_per_block; /* attention kernel */
  int32_t lds_bytes;         /* attention kernel: LDS per workgroup, static + dynamic */
  int32_t parents_in_lds;    /* in-kernel walk: parent rows copied to LDS first */
  int32_t beams_per_block;   /* staged kernel, in-kernel walk: most beams one
                                workgroup's query rows belong to */
  int64_t grid;              /* attention kernel workgroups */
  size_t workspace_bytes;    /* xattn_workspace_size(shape, step) */
} xattn_plan;

/* Fills *plan for xattn_decode(shape, ..., step, ...).  Returns the status
 * xattn_decode would return for the shape and step (XATTN_EINVAL for a bad
 * shape, step or NULL plan; XATTN_EUNSUPPORTED where no kernel fits). */
xattn_status xattn_plan_decode(const xattn_shape *shape, int32_t step, xattn_plan *plan);

/* Static description of a status code. */
const char *xattn_status_string(xattn_status status);

/* Reason for the calling thread's most recent non-OK status ("" if none). */
const char *xattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
