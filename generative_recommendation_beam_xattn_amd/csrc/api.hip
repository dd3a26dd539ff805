// C ABI of libxattn.so (declared in include/xattn.h): argument validation,
// tiling choice and kernel dispatch on the caller's stream.  Nothing here
// touches device memory; every check below runs before anything is enqueued.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/xattn.h"
#include "../../include/xattn_measure.h"
#include "../../include/xbeam.h"
#include "xattn_internal.h"

namespace {

thread_local char g_last_error[256] = "";

xattn_status fail(xattn_status st, const char *msg) {
  snprintf(g_last_error, sizeof g_last_error, "%s", msg);
  return st;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;  // per tensor, keeps 64-bit offsets far from overflow

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

xattn_status check_shape(const xattn_shape *s, int32_t step) {
  if (!s) return fail(XATTN_EINVAL, "shape is NULL");
  if (s->num_requests < 1) return fail(XATTN_EINVAL, "num_requests must be >= 1");
  if (s->beam_width < 1) return fail(XATTN_EINVAL, "beam_width must be >= 1");
  if (s->num_kv_heads < 1 || s->num_q_heads < 1)
    return fail(XATTN_EINVAL, "head counts must be >= 1");
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(XATTN_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (s->max_prompt_len < 0) return fail(XATTN_EINVAL, "max_prompt_len must be >= 0");
  if (s->max_steps < 1) return fail(XATTN_EINVAL, "max_steps must be >= 1");
  if (step < 0 || step >= s->max_steps) return fail(XATTN_EINVAL, "step must be in [0, max_steps)");
  if (!(s->scale >= 0.f) || !isfinite(s->scale))
    return fail(XATTN_EINVAL, "scale must be finite and >= 0");
  if (s->dtype != XATTN_F32 && s->dtype != XATTN_BF16) return fail(XATTN_EINVAL, "unknown dtype");
  if (s->head_dim < 1) return fail(XATTN_EINVAL, "head_dim must be >= 1");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(XATTN_EUNSUPPORTED, "head_dim must be 64 or 128");
  const int64_t R = s->num_requests, BW = s->beam_width, Hq = s->num_q_heads,
                Hkv = s->num_kv_heads, D = s->head_dim, Lmax = s->max_prompt_len,
                S = s->max_steps;
  const double q_elems = (double)R * BW * Hq * D;
  const double sh_elems = (double)R * Hkv * Lmax * D;
  const double un_elems = (double)R * Hkv * S * BW * D;
  const double par_elems = (double)R * S * BW;
  if (q_elems > kMaxElems || sh_elems > kMaxElems || un_elems > kMaxElems || par_elems > kMaxElems)
    return fail(XATTN_EINVAL, "a tensor exceeds 2^40 elements");
  if ((double)BW * (Hq / Hkv) > 0x7fffffff) return fail(XATTN_EINVAL, "beam_width * group too large");
  return XATTN_OK;
}

bool deep_chain(int32_t step) { return step + 1 > xattn::kMaxInKernelLevels; }

// Workspace of a deep-chain call: the resolved ancestor slots, the composed
// parent maps of the segmented walk (long chains), then (bf16) the
// Unshared-stage partials of every query row, (m, l) and o [D] in float,
// and the key splits' partials.
size_t anc_bytes_for(const xattn_shape *s, int32_t step) {
  const size_t n = (size_t)s->num_requests * (size_t)(step + 1) * (size_t)s->beam_width;
  return (n * sizeof(int32_t) + 255) & ~size_t(255);
}

size_t seg_map_bytes_for(const xattn_shape *s, int32_t step) {
  const int lps = xattn::ancestor_segment_levels(s->beam_width, step);
  if (lps == 0) return 0;
  const size_t n = (size_t)s->num_requests * (size_t)((step + lps - 1) / lps) *
                   (size_t)s->beam_width;
  return (n * sizeof(int32_t) + 255) & ~size_t(255);
}

size_t rows_of(const xattn_shape *s) {
  return (size_t)s->num_requests * (size_t)s->beam_width * (size_t)s->num_q_heads;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Key splits of a deep-chain bf16 call on the staged kernel: when its
// (request, KV head, row block) workgroups cannot fill the GPU's 256
// compute units, each one's prompt tiles are split over up to 4
// workgroups (at least 4 tiles each), whose partials a merge kernel
// combines.  A function of the shape alone, so that xattn_workspace_size
// can count the partials.
int key_splits_for(const xattn_shape *s, int32_t step) {
  if (!deep_chain(step) || s->dtype != XATTN_BF16) return 1;
  const int64_t M = (int64_t)s->beam_width * (s->num_q_heads / s->num_kv_heads);
  if (M <= xattn::kPerBeamMaxRows) return 1;   // runs on the per-beam kernel
  xattn::DecodeParams p{};
  p.M = (int32_t)M;
  const int64_t rows = xattn::bf16_rows_per_block(p);
  const int64_t grid = (int64_t)s->num_requests * s->num_kv_heads * ((M + rows - 1) / rows);
  if (grid >= 128) return 1;
  const int64_t tiles = ((int64_t)s->max_prompt_len + 63) / 64;
  const int64_t n = std::min<int64_t>({xattn::kMaxKeySplits, 256 / grid, tiles / 4});
  return n >= 2 ? (int)n : 1;
}

size_t workspace_bytes_for(const xattn_shape *s, int32_t step) {
  if (!deep_chain(step)) return 0;
  size_t bytes = anc_bytes_for(s, step) + seg_map_bytes_for(s, step);
  if (s->dtype == XATTN_BF16) {
    bytes += round256(rows_of(s) * 2 * sizeof(float));
    bytes += round256(rows_of(s) * (size_t)s->head_dim * sizeof(float));
    const size_t ns = (size_t)key_splits_for(s, step);
    if (ns > 1) {
      bytes += round256(ns * rows_of(s) * 2 * sizeof(float));
      bytes += round256(ns * rows_of(s) * (size_t)s->head_dim * sizeof(float));
    }
  }
  return bytes;
}

// What one decode call enqueues for this shape and step (xattn_plan in
// include/xattn.h): the plan the dispatch below follows, computed on the
// host alone.
enum Walk { kWalkInKernel = 0, kWalkChunked = 1, kWalkSegmented = 2 };

xattn_status make_plan(const xattn_shape *s, int32_t step, bool per_beam, bool taps,
                       xattn_plan *pl) {
  xattn_status st = check_shape(s, step);
  if (st != XATTN_OK) return st;
  memset(pl, 0, sizeof *pl);
  const bool deep = deep_chain(step);
  const int64_t G = s->num_q_heads / s->num_kv_heads;
  const int64_t M = (int64_t)s->beam_width * G;
  const bool staged_bf16 =
      s->dtype == XATTN_BF16 && !per_beam && (taps || M > xattn::kPerBeamMaxRows);
  pl->workspace_bytes = workspace_bytes_for(s, step);
  pl->ancestor_walk = !deep ? kWalkInKernel
                            : (seg_map_bytes_for(s, step) > 0 ? kWalkSegmented : kWalkChunked);
  pl->kernel = s->dtype == XATTN_F32 ? XATTN_KERNEL_F32
                                     : (staged_bf16 ? XATTN_KERNEL_STAGED_BF16
                                                    : XATTN_KERNEL_PER_BEAM_BF16);
  pl->key_splits = staged_bf16 && !taps ? key_splits_for(s, step) : 1;
  pl->unshared_kernel = deep && staged_bf16 ? 1 : 0;
  pl->kernels = (pl->ancestor_walk == kWalkSegmented ? 2 : (deep ? 1 : 0)) +
                pl->unshared_kernel + 1 + (pl->key_splits > 1 ? 1 : 0);
  if (staged_bf16) {
    xattn::DecodeParams p{};
    p.R = s->num_requests;
    p.BW = s->beam_width;
    p.Hq = s->num_q_heads;
    p.Hkv = s->num_kv_heads;
    p.D = s->head_dim;
    p.step = step;
    p.G = (int32_t)G;
    p.M = (int32_t)M;
    p.n_split = pl->key_splits;
    static const int32_t resolved = 0;   // any non-null: slots come from the workspace
    p.anc = deep ? &resolved : nullptr;
    const xattn::Bf16Geometry g = xattn::bf16_geometry(p);
    if (g.paired) pl->kernel = XATTN_KERNEL_STAGED_BF16_PAIRED;
    pl->rows_per_block = g.rows;
    pl->threads_per_block = g.threads;
    pl->grid = g.grid;
    pl->lds_bytes = g.static_lds + g.dyn_lds;
    pl->parents_in_lds = g.stage_par ? 1 : 0;
    pl->beams_per_block = deep ? 0 : g.beams_per_block;
  } else if (s->dtype == XATTN_F32) {
    pl->rows_per_block = 1;
    pl->threads_per_block = xattn::kF32Threads;
    pl->grid = (int64_t)s->num_requests * s->beam_width * s->num_q_heads;
    pl->lds_bytes = xattn::f32_lds_bytes(s->head_dim);
  } else {
    pl->rows_per_block = (int32_t)G;
    pl->threads_per_block = xattn::kPerBeamThreads;
    pl->grid = (int64_t)s->num_requests * s->beam_width * s->num_kv_heads;
    pl->lds_bytes = xattn::per_beam_lds_bytes(s->head_dim);
  }
  if (pl->grid > 0x7fffffff) return fail(XATTN_EUNSUPPORTED, "too many workgroups for one launch");
  if (pl->lds_bytes > xattn::kLdsLimit)
    return fail(XATTN_EUNSUPPORTED, "the kernel's LDS does not fit this shape");
  return XATTN_OK;
}

// Optional outputs and modes of one decode call.
struct RunOpts {
  float *lse = nullptr;          // debug taps
  float *stage_ml = nullptr;
  float *stage_o = nullptr;
  int32_t *anc_out = nullptr;    // ancestor slots [R][step+1][BW]
  bool want_anc = false;         // anc_out is a required argument
  bool taps = false;             // debug entry: stages kept apart
  bool per_beam = false;         // the per-beam comparison kernel
  xattn::LaunchEvents ev{};
};

xattn_status run(const xattn_shape *s, const void *q, const void *shared_k, const void *shared_v,
                 const int32_t *prompt_len, const void *unshared_k, const void *unshared_v,
                 const int32_t *parent_idx, int32_t step, void *out, void *workspace,
                 size_t workspace_bytes, void *stream, const RunOpts &o) {
  xattn_plan pl;
  xattn_status st = make_plan(s, step, o.per_beam, o.taps, &pl);
  if (st != XATTN_OK) return st;
  if (!q || !prompt_len || !unshared_k || !unshared_v || !parent_idx || !out ||
      (o.want_anc && !o.anc_out))
    return fail(XATTN_EINVAL, "a required pointer is NULL");
  if (s->max_prompt_len > 0 && (!shared_k || !shared_v))
    return fail(XATTN_EINVAL, "shared_k/shared_v are NULL but max_prompt_len > 0");
  const void *vec[] = {q, shared_k, shared_v, unshared_k, unshared_v, out};
  for (const void *v : vec)
    if (!aligned(v, 16)) return fail(XATTN_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (!aligned(prompt_len, 4) || !aligned(parent_idx, 4))
    return fail(XATTN_EINVAL, "int32 arrays must be 4-byte aligned");
  if ((o.lse && !aligned(o.lse, 4)) || (o.stage_ml && !aligned(o.stage_ml, 4)) ||
      (o.stage_o && !aligned(o.stage_o, 4)) || (o.anc_out && !aligned(o.anc_out, 4)))
    return fail(XATTN_EINVAL, "tap arrays must be 4-byte aligned");
  const size_t need = pl.workspace_bytes;
  if (need > 0) {
    if (!workspace) return fail(XATTN_EINVAL, "this step needs a workspace (xattn_workspace_size)");
    if (workspace_bytes < need) return fail(XATTN_EINVAL, "workspace is smaller than xattn_workspace_size");
    if (!aligned(workspace, 256)) return fail(XATTN_EINVAL, "workspace must be 256-byte aligned");
  }

  xattn::DecodeParams p{};
  p.q = q;
  p.shared_k = shared_k;
  p.shared_v = shared_v;
  p.prompt_len = prompt_len;
  p.unshared_k = unshared_k;
  p.unshared_v = unshared_v;
  p.parent_idx = parent_idx;
  p.out = out;
  p.lse = o.lse;
  p.stage_ml = o.stage_ml;
  p.stage_o = o.stage_o;
  p.anc_out = o.anc_out;
  p.R = s->num_requests;
  p.BW = s->beam_width;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.D = s->head_dim;
  p.Lmax = s->max_prompt_len;
  p.S = s->max_steps;
  p.step = step;
  p.G = p.Hq / p.Hkv;
  p.M = p.BW * p.G;
  p.scale = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)p.D);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  // the debug taps report each stage's true maximum
  p.lazy_log2 = o.taps ? 0.f : xattn::kLazyRescaleLog2;
  p.n_split = 1;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // timing events: start bound to the call's first kernel, stop to its last
  int launched = 0;
  auto evs = [&]() {
    xattn::LaunchEvents r{launched == 0 ? o.ev.start : nullptr,
                          launched == pl.kernels - 1 ? o.ev.stop : nullptr};
    ++launched;
    return r;
  };
  if (pl.ancestor_walk != kWalkInKernel) {
    int32_t *anc = static_cast<int32_t *>(workspace);
    const xattn::AncLayout lay{(int64_t)(step + 1) * p.BW, 1, p.BW};  // [R][step+1][BW]
    if (pl.ancestor_walk == kWalkSegmented) {
      int32_t *fmap = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) +
                                                  anc_bytes_for(s, step));
      // both walk kernels go in the call's timing window
      xattn::LaunchEvents ev_walk{launched == 0 ? o.ev.start : nullptr, nullptr};
      launched += 2;
      e = xattn::launch_resolve_ancestors_segmented(parent_idx, p.R, p.BW, p.S, step, anc, lay,
                                                    fmap, hs, ev_walk);
    } else {
      e = xattn::launch_resolve_ancestors(parent_idx, p.R, p.BW, p.S, step, anc, lay, hs, evs());
    }
    if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
    p.anc = anc;
    if (o.anc_out) {
      // the slots the walk kernels wrote, in the same layout
      e = hipMemcpyAsync(o.anc_out, anc, (size_t)p.R * (step + 1) * p.BW * sizeof(int32_t),
                         hipMemcpyDeviceToDevice, hs);
      if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
    }
  }
  if (pl.unshared_kernel) {
    // deep chains: the Unshared stage runs first with one workgroup per
    // (request, beam, KV head), so the gather of every beam's token rows
    // spreads over the whole GPU; the staged kernel starts from its partials
    uint8_t *w = static_cast<uint8_t *>(workspace) + anc_bytes_for(s, step) +
                 seg_map_bytes_for(s, step);
    p.tok_ml = reinterpret_cast<float *>(w);
    w += round256(rows_of(s) * 2 * sizeof(float));
    p.tok_o = reinterpret_cast<float *>(w);
    w += round256(rows_of(s) * (size_t)s->head_dim * sizeof(float));
    if (pl.key_splits > 1) {
      p.n_split = pl.key_splits;
      p.part_ml = reinterpret_cast<float *>(w);
      w += round256((size_t)pl.key_splits * rows_of(s) * 2 * sizeof(float));
      p.part_o = reinterpret_cast<float *>(w);
    }
    e = xattn::launch_token_partials_bf16(p, hs, evs());
    if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  }
  const xattn::LaunchEvents ev_main = evs();
  if (pl.kernel == XATTN_KERNEL_F32)
    e = xattn::launch_decode_f32(p, hs, ev_main);  // per query row already: also the per-beam form
  else if (pl.kernel == XATTN_KERNEL_PER_BEAM_BF16)
    e = xattn::launch_decode_per_beam_bf16(p, hs, ev_main);
  else
    e = xattn::launch_decode_bf16(p, o.taps, hs, ev_main);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  if (pl.key_splits > 1) {
    e = xattn::launch_merge_splits_bf16(p, hs, evs());
    if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  }
  g_last_error[0] = '\0';
  return XATTN_OK;
}

// ---- device scratch of xattn_decode_noalloc: one file-scope array, which
// each GPU the library runs on holds (its own copy, at its own address)
// until the process ends.  Host code never uses the array's name as an
// address: it takes each device's address once, with that device current,
// and passes that.
constexpr size_t kScratchBytes = size_t(XATTN_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up on its first
// use on that device).
xattn_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(XATTN_EUNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
    if (!p || !aligned(p, 256)) return fail(XATTN_EHIP, "scratch address is not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return XATTN_OK;
}

xattn_status beam_topk(const float *cum, const float *logp, const int32_t *token, int32_t R,
                       int32_t BW, int32_t V, float *new_score, int32_t *new_parent,
                       int32_t *new_token, int64_t out_stride, void *stream,
                       xattn::LaunchEvents ev = {}) {
  if (R < 1) return fail(XATTN_EINVAL, "R must be >= 1");
  if (BW < 1 || BW > XBEAM_MAX_BEAMS) return fail(XATTN_EINVAL, "BW must be in [1, 512]");
  if (V < 1 || V > (1 << 24)) return fail(XATTN_EINVAL, "V must be in [1, 2^24]");
  if (out_stride < BW) return fail(XATTN_EINVAL, "out_stride must be >= BW");
  if ((double)R * BW * V > kMaxElems || (double)R * out_stride > kMaxElems)
    return fail(XATTN_EINVAL, "an array exceeds 2^40 elements");
  if (!cum || !logp || !token || !new_score || !new_parent || !new_token)
    return fail(XATTN_EINVAL, "a required pointer is NULL");
  const void *ptrs[] = {cum, logp, token, new_score, new_parent, new_token};
  for (const void *v : ptrs)
    if (!aligned(v, 4)) return fail(XATTN_EINVAL, "arrays must be 4-byte aligned");
  static_assert(XBEAM_MAX_BEAMS == xattn::kMaxTopkBeams, "beam limit mismatch");
  hipError_t e = xattn::launch_beam_topk(cum, logp, token, R, BW, V, new_score, new_parent,
                                         new_token, out_stride, static_cast<hipStream_t>(stream),
                                         ev);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return XATTN_OK;
}

xattn_status reorder_unshared(const xattn_shape *s, void *unshared_k, void *unshared_v,
                              const int32_t *parent, int64_t parent_stride, int32_t n_levels,
                              void *stream, xattn::LaunchEvents ev = {}) {
  xattn_status st = check_shape(s, 0);
  if (st != XATTN_OK) return st;
  if (n_levels < 0 || n_levels > s->max_steps)
    return fail(XATTN_EINVAL, "n_levels must be in [0, max_steps]");
  if (!unshared_k || !unshared_v || !parent) return fail(XATTN_EINVAL, "a required pointer is NULL");
  if (!aligned(unshared_k, 16) || !aligned(unshared_v, 16))
    return fail(XATTN_EINVAL, "unshared_k/unshared_v must be 16-byte aligned");
  if (!aligned(parent, 4)) return fail(XATTN_EINVAL, "int32 arrays must be 4-byte aligned");
  if (parent_stride < s->beam_width) return fail(XATTN_EINVAL, "parent_stride must be >= beam_width");
  if ((double)s->num_requests * parent_stride > kMaxElems)
    return fail(XATTN_EINVAL, "parent rows exceed 2^40 elements");
  if (s->beam_width > xattn::kMaxReorderBeams)
    return fail(XATTN_EUNSUPPORTED, "beam_width above 2048 is not supported by the reorder");
  xattn::ReorderParams p{};
  p.unshared_k = unshared_k;
  p.unshared_v = unshared_v;
  p.parent = parent;
  p.parent_stride = parent_stride;
  p.row_bytes = (int64_t)s->head_dim * (s->dtype == XATTN_F32 ? 4 : 2);
  p.chunk_bytes = xattn::reorder_chunk_bytes(p.row_bytes, s->beam_width);
  p.R = s->num_requests;
  p.Hkv = s->num_kv_heads;
  p.S = s->max_steps;
  p.BW = s->beam_width;
  p.n_levels = n_levels;
  hipError_t e = xattn::launch_reorder_unshared(p, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return XATTN_OK;
}

xattn_status check_trie(const xattn_trie *lay, const void *table, int32_t depth) {
  if (!lay || !table) return fail(XATTN_EINVAL, "layout and table are required");
  if (lay->levels < 1 || lay->levels > XATTN_TRIE_MAX_LEVELS || lay->vocab < 1 ||
      lay->vocab > 32 * xattn::kMaxMaskWords || lay->words != (lay->vocab + 31) / 32 ||
      lay->dense_levels < 0 || lay->dense_levels > lay->levels)
    return fail(XATTN_EINVAL, "layout is not one xattn_trie_build wrote");
  if (depth < 0 || depth >= lay->levels) return fail(XATTN_EINVAL, "depth must be in [0, levels)");
  if (!aligned(table, 256)) return fail(XATTN_EINVAL, "table must be 256-byte aligned");
  return XATTN_OK;
}

xattn_status valid_mask(const xattn_trie *lay, const void *table, int32_t depth,
                        const int32_t *node, float *logits, int32_t R, int32_t BW,
                        int64_t row_stride, void *stream, xattn::LaunchEvents ev = {}) {
  xattn_status st = check_trie(lay, table, depth);
  if (st != XATTN_OK) return st;
  if (R < 1 || BW < 1) return fail(XATTN_EINVAL, "R and BW must be >= 1");
  if (!node || !logits) return fail(XATTN_EINVAL, "a required pointer is NULL");
  if (row_stride < lay->vocab || row_stride % 4 != 0)
    return fail(XATTN_EINVAL, "row_stride must be >= vocab and a multiple of 4");
  if ((double)R * BW * row_stride > kMaxElems) return fail(XATTN_EINVAL, "logits exceed 2^40 elements");
  if (!aligned(logits, 16)) return fail(XATTN_EINVAL, "logits must be 16-byte aligned");
  if (!aligned(node, 4)) return fail(XATTN_EINVAL, "int32 arrays must be 4-byte aligned");
  xattn::MaskParams p{};
  p.table = static_cast<const uint8_t *>(table);
  p.node = node;
  p.logits = logits;
  p.row_stride = row_stride;
  p.row_ptr_off = lay->row_ptr_off[depth];
  p.child_tok_off = lay->child_tok_off[depth];
  p.mask_off = depth < lay->dense_levels ? lay->mask_off[depth] : 0;
  p.R = R;
  p.BW = BW;
  p.V = lay->vocab;
  p.words = lay->words;
  p.n_nodes = lay->nodes[depth];
  p.n_edges = lay->nodes[depth + 1];
  p.dense = depth < lay->dense_levels ? 1 : 0;
  hipError_t e = xattn::launch_valid_mask(p, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return XATTN_OK;
}

}  // namespace

extern "C" {

xattn_status xattn_trie_build(const int32_t *items, int64_t n_items, int32_t levels,
                              int32_t vocab, int32_t dense_levels, xattn_trie *layout,
                              void *host_table, size_t host_bytes) {
  if (!layout) return fail(XATTN_EINVAL, "layout is NULL");
  const char *err = xattn::build_trie(items, n_items, levels, vocab, dense_levels, layout,
                                      host_table, host_bytes);
  if (err) return fail(XATTN_EINVAL, err);
  g_last_error[0] = '\0';
  return XATTN_OK;
}

xattn_status xattn_valid_mask(const xattn_trie *layout, const void *table, int32_t depth,
                              const int32_t *node, float *logits, int32_t R, int32_t BW,
                              int64_t row_stride, void *stream) {
  return valid_mask(layout, table, depth, node, logits, R, BW, row_stride, stream);
}

xattn_status xattn_valid_mask_timed(const xattn_trie *layout, const void *table, int32_t depth,
                                    const int32_t *node, float *logits, int32_t R, int32_t BW,
                                    int64_t row_stride, void *stream, void *start_event,
                                    void *stop_event) {
  if (!start_event || !stop_event) return fail(XATTN_EINVAL, "both timing events are required");
  xattn::LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  return valid_mask(layout, table, depth, node, logits, R, BW, row_stride, stream, ev);
}

xattn_status xattn_trie_advance(const xattn_trie *layout, const void *table, int32_t depth,
                                const int32_t *node, const int32_t *parent,
                                int64_t parent_stride, const int32_t *token,
                                int64_t token_stride, int32_t *new_node, int32_t R, int32_t BW,
                                void *stream) {
  xattn_status st = check_trie(layout, table, depth);
  if (st != XATTN_OK) return st;
  if (R < 1 || BW < 1) return fail(XATTN_EINVAL, "R and BW must be >= 1");
  if (!node || !parent || !token || !new_node) return fail(XATTN_EINVAL, "a required pointer is NULL");
  if (parent_stride < BW || token_stride < BW)
    return fail(XATTN_EINVAL, "parent_stride and token_stride must be >= BW");
  if ((double)R * parent_stride > kMaxElems || (double)R * token_stride > kMaxElems ||
      (double)R * BW > kMaxElems)
    return fail(XATTN_EINVAL, "an array exceeds 2^40 elements");
  const void *ptrs[] = {node, parent, token, new_node};
  for (const void *v : ptrs)
    if (!aligned(v, 4)) return fail(XATTN_EINVAL, "int32 arrays must be 4-byte aligned");
  xattn::AdvanceParams p{};
  p.table = static_cast<const uint8_t *>(table);
  p.node = node;
  p.parent = parent;
  p.parent_stride = parent_stride;
  p.token = token;
  p.token_stride = token_stride;
  p.new_node = new_node;
  p.row_ptr_off = layout->row_ptr_off[depth];
  p.child_tok_off = layout->child_tok_off[depth];
  p.R = R;
  p.BW = BW;
  p.V = layout->vocab;
  p.n_nodes = layout->nodes[depth];
  p.n_edges = layout->nodes[depth + 1];
  hipError_t e = xattn::launch_trie_advance(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return XATTN_OK;
}

xattn_status xattn_reorder_unshared(const xattn_shape *shape, void *unshared_k, void *unshared_v,
                                    const int32_t *parent, int64_t parent_stride,
                                    int32_t n_levels, void *stream) {
  return reorder_unshared(shape, unshared_k, unshared_v, parent, parent_stride, n_levels, stream);
}

xattn_status xattn_reorder_unshared_timed(const xattn_shape *shape, void *unshared_k,
                                          void *unshared_v, const int32_t *parent,
                                          int64_t parent_stride, int32_t n_levels, void *stream,
                                          void *start_event, void *stop_event) {
  if (!start_event || !stop_event) return fail(XATTN_EINVAL, "both timing events are required");
  xattn::LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  return reorder_unshared(shape, unshared_k, unshared_v, parent, parent_stride, n_levels, stream,
                          ev);
}

xattn_status xattn_beam_topk(const float *cum, const float *logp, const int32_t *token,
                             int32_t R, int32_t BW, int32_t V, float *new_score,
                             int32_t *new_parent, int32_t *new_token, int64_t out_stride,
                             void *stream) {
  return beam_topk(cum, logp, token, R, BW, V, new_score, new_parent, new_token, out_stride,
                   stream);
}

xattn_status xattn_beam_topk_timed(const float *cum, const float *logp, const int32_t *token,
                                   int32_t R, int32_t BW, int32_t V, float *new_score,
                                   int32_t *new_parent, int32_t *new_token, int64_t out_stride,
                                   void *stream, void *start_event, void *stop_event) {
  if (!start_event || !stop_event) return fail(XATTN_EINVAL, "both timing events are required");
  xattn::LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  return beam_topk(cum, logp, token, R, BW, V, new_score, new_parent, new_token, out_stride,
                   stream, ev);
}

xattn_status xattn_decode(const xattn_shape *shape, const void *q, const void *shared_k,
                          const void *shared_v, const int32_t *prompt_len,
                          const void *unshared_k, const void *unshared_v,
                          const int32_t *parent_idx, int32_t step, void *out, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, workspace, workspace_bytes, stream, RunOpts{});
}

xattn_status xattn_decode_noalloc(const xattn_shape *shape, const void *q, const void *shared_k,
                                  const void *shared_v, const int32_t *prompt_len,
                                  const void *unshared_k, const void *unshared_v,
                                  const int32_t *parent_idx, int32_t step, void *out,
                                  void *stream) {
  xattn_plan pl;
  xattn_status st = make_plan(shape, step, false, false, &pl);
  if (st != XATTN_OK) return st;
  if (pl.workspace_bytes == 0)
    return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
               out, nullptr, 0, stream, RunOpts{});
  if (pl.workspace_bytes > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "this step needs %zu bytes of workspace, more than the %zu-byte scratch of "
             "xattn_decode_noalloc; use xattn_decode with a workspace",
             pl.workspace_bytes, kScratchBytes);
    return fail(XATTN_EINVAL, msg);
  }
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != XATTN_OK) return st;
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, ws, kScratchBytes, stream, RunOpts{});
}

xattn_status xattn_decode_with_ancestors(const xattn_shape *shape, const void *q,
                                         const void *shared_k, const void *shared_v,
                                         const int32_t *prompt_len, const void *unshared_k,
                                         const void *unshared_v, const int32_t *parent_idx,
                                         int32_t step, void *out, int32_t *anc, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  RunOpts o;
  o.anc_out = anc;
  o.want_anc = true;
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, workspace, workspace_bytes, stream, o);
}

xattn_status xattn_decode_debug(const xattn_shape *shape, const void *q, const void *shared_k,
                                const void *shared_v, const int32_t *prompt_len,
                                const void *unshared_k, const void *unshared_v,
                                const int32_t *parent_idx, int32_t step, void *out, float *lse,
                                float *stage_ml, float *stage_o, void *workspace,
                                size_t workspace_bytes, void *stream) {
  RunOpts o;
  o.lse = lse;
  o.stage_ml = stage_ml;
  o.stage_o = stage_o;
  o.taps = true;
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, workspace, workspace_bytes, stream, o);
}

xattn_status xattn_decode_timed(const xattn_shape *shape, const void *q, const void *shared_k,
                                const void *shared_v, const int32_t *prompt_len,
                                const void *unshared_k, const void *unshared_v,
                                const int32_t *parent_idx, int32_t step, void *out,
                                void *workspace, size_t workspace_bytes, void *stream,
                                void *start_event, void *stop_event) {
  if (!start_event || !stop_event) return fail(XATTN_EINVAL, "both timing events are required");
  RunOpts o;
  o.ev.start = static_cast<hipEvent_t>(start_event);
  o.ev.stop = static_cast<hipEvent_t>(stop_event);
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, workspace, workspace_bytes, stream, o);
}

xattn_status xattn_decode_per_beam(const xattn_shape *shape, const void *q, const void *shared_k,
                                   const void *shared_v, const int32_t *prompt_len,
                                   const void *unshared_k, const void *unshared_v,
                                   const int32_t *parent_idx, int32_t step, void *out,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  RunOpts o;
  o.per_beam = true;
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, workspace, workspace_bytes, stream, o);
}

xattn_status xattn_decode_per_beam_timed(const xattn_shape *shape, const void *q,
                                         const void *shared_k, const void *shared_v,
                                         const int32_t *prompt_len, const void *unshared_k,
                                         const void *unshared_v, const int32_t *parent_idx,
                                         int32_t step, void *out, void *workspace,
                                         size_t workspace_bytes, void *stream, void *start_event,
                                         void *stop_event) {
  if (!start_event || !stop_event) return fail(XATTN_EINVAL, "both timing events are required");
  RunOpts o;
  o.per_beam = true;
  o.ev.start = static_cast<hipEvent_t>(start_event);
  o.ev.stop = static_cast<hipEvent_t>(stop_event);
  return run(shape, q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
             out, workspace, workspace_bytes, stream, o);
}

xattn_status xattn_plan_decode(const xattn_shape *shape, int32_t step, xattn_plan *plan) {
  if (!plan) return fail(XATTN_EINVAL, "plan is NULL");
  const xattn_status st = make_plan(shape, step, false, false, plan);
  if (st == XATTN_OK) g_last_error[0] = '\0';
  return st;
}

size_t xattn_workspace_size(const xattn_shape *shape, int32_t step) {
  if (check_shape(shape, step) != XATTN_OK) return (size_t)-1;
  return workspace_bytes_for(shape, step);
}

xattn_status xattn_resolve_ancestors(const xattn_shape *shape, const int32_t *parent_idx,
                                     int32_t step, int32_t *anc, void *stream) {
  xattn_status st = check_shape(shape, step);
  if (st != XATTN_OK) return st;
  if (!parent_idx || !anc) return fail(XATTN_EINVAL, "a required pointer is NULL");
  if (!aligned(parent_idx, 4) || !aligned(anc, 4))
    return fail(XATTN_EINVAL, "int32 arrays must be 4-byte aligned");
  const int32_t BW = shape->beam_width;
  const xattn::AncLayout lay{(int64_t)BW * (step + 1), step + 1, 1};  // [R][BW][step+1]
  hipError_t e = xattn::launch_resolve_ancestors(parent_idx, shape->num_requests, BW,
                                                 shape->max_steps, step, anc, lay,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return XATTN_OK;
}

const char *xattn_status_string(xattn_status status) {
  switch (status) {
    case XATTN_OK: return "ok";
    case XATTN_EINVAL: return "invalid argument";
    case XATTN_EUNSUPPORTED: return "unsupported shape or dtype";
    case XATTN_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *xattn_last_error(void) { return g_last_error; }

xattn_status xattn_peak_mfma_bf16(int32_t iters, int32_t blocks, float *out, void *stream,
                                  void *start_event, void *stop_event, double *flops) {
  if (iters < 1 || blocks < 1) return fail(XATTN_EINVAL, "iters and blocks must be >= 1");
  if (!out || !aligned(out, 4)) return fail(XATTN_EINVAL, "out must be a 4-byte-aligned device buffer");
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(XATTN_EINVAL, "give both timing events or neither");
  xattn::LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  const hipError_t e =
      xattn::launch_peak_mfma(iters, blocks, out, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  if (flops) *flops = xattn::peak_mfma_flops(iters, blocks);
  g_last_error[0] = '\0';
  return XATTN_OK;
}

xattn_status xattn_peak_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *out,
                             void *stream, void *start_event, void *stop_event) {
  if (blocks < 1 || bytes < 16 || bytes % 16 != 0)
    return fail(XATTN_EINVAL, "blocks must be >= 1 and bytes a positive multiple of 16");
  if (!src || !aligned(src, 16)) return fail(XATTN_EINVAL, "src must be a 16-byte-aligned device buffer");
  if (!out || !aligned(out, 4)) return fail(XATTN_EINVAL, "out must be a 4-byte-aligned device buffer");
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(XATTN_EINVAL, "give both timing events or neither");
  xattn::LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  const hipError_t e =
      xattn::launch_peak_read(src, bytes, blocks, out, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return fail(XATTN_EHIP, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return XATTN_OK;
}

}  // extern "C"
