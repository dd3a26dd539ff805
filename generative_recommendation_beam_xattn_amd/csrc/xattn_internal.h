// Internal declarations of libxattn.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/xbeam.h"

namespace xattn {

// Chains of at most this many levels are walked inside the attention kernel
// (slots kept in LDS); deeper chains are resolved by the ancestor kernel into
// the workspace first.
constexpr int kMaxInKernelLevels = 16;

// With this few query rows per (request, KV head) -- one or two beams -- the
// staged kernel's 32-row MFMA blocks are mostly empty and there is almost
// nothing to share; the per-beam kernel runs those calls (measured on the
// prefix-sharing shapes: 1079 vs 2903 us at 4 rows, 957 vs 1498 us at 8,
// and the staged kernel ahead from 16 rows).
constexpr int kPerBeamMaxRows = 8;
// Most key splits one staged workgroup's prompt tiles are spread over.
constexpr int kMaxKeySplits = 4;
// On the decode path a running maximum is raised only when a score exceeds
// it by more than 2^8 in the exp2 domain (DecodeParams::lazy_log2).
constexpr float kLazyRescaleLog2 = 8.0f;

// Largest beam width the beam-selection kernel takes.
constexpr int kMaxTopkBeams = 512;
// Largest beam width the Unshared-cache reorder takes.
constexpr int kMaxReorderBeams = 2048;

// Optional pair of events bound to kernel dispatches (hipExtLaunchKernel):
// start is recorded as the dispatch begins and stop as it ends; a call of
// several kernels binds start to its first and stop to its last.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Everything a decode launch needs; passed by value as a kernel argument.
struct DecodeParams {
  const void *q;
  const void *shared_k;
  const void *shared_v;
  const int32_t *prompt_len;
  const void *unshared_k;
  const void *unshared_v;
  const int32_t *parent_idx;
  void *out;
  const int32_t *anc;  // [R][step+1][BW] resolved slots, or nullptr: walk in-kernel
  float *tok_ml;       // deep chains: Unshared-stage partials per query row,
  float *tok_o;        // (m, l) and unnormalised o [D], computed beforehand
  float *part_ml;      // key splits (n_split > 1): per split and query row the
  float *part_o;       // partial (m, l) and unnormalised o [D], merged afterwards
  float *lse;          // optional taps (debug entry only)
  float *stage_ml;
  float *stage_o;
  int32_t *anc_out;    // optional [R][step+1][BW]: the ancestor slots the
                       // Unshared stage gathered, written by the walking kernel
  int32_t R, BW, Hq, Hkv, D, Lmax, S, step;
  int32_t G;           // Hq / Hkv, query heads per KV head
  int32_t M;           // BW * G query rows per (request, KV head)
  int32_t n_rb;        // row blocks per (request, KV head)
  int32_t n_split;     // key splits of the prompt per row block (1: none)
  int32_t stage_par;   // bf16 in-kernel walk: 1 = parent rows copied to LDS first
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e): scores go through exp2
  float lazy_log2;     // a running maximum moves only when a score exceeds it by
                       // more than this (exp2 units); 0 keeps the exact maximum
};

// Ancestor output layouts: element (r, b, t) lives at
//   r * stride_r + b * stride_b + t * stride_t.
struct AncLayout {
  int64_t stride_r, stride_b, stride_t;
};


hipError_t launch_resolve_ancestors(const int32_t *parent_idx, int32_t R, int32_t BW, int32_t S,
                                    int32_t step, int32_t *anc, AncLayout layout,
                                    hipStream_t stream, LaunchEvents ev = {});
// Long chains: levels per segment of the two-kernel segmented walk, or 0
// when it does not apply (one segment, or too many slots for LDS).  fmap
// holds R * ceil(step / levels) * BW int32 of composed segment maps.
int ancestor_segment_levels(int32_t BW, int32_t step);
hipError_t launch_resolve_ancestors_segmented(const int32_t *parent_idx, int32_t R, int32_t BW,
                                              int32_t S, int32_t step, int32_t *anc,
                                              AncLayout layout, int32_t *fmap,
                                              hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_decode_bf16(const DecodeParams &p, bool taps, hipStream_t stream,
                              LaunchEvents ev = {});
hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_decode_per_beam_bf16(const DecodeParams &p, hipStream_t stream,
                                       LaunchEvents ev = {});
// Matrix-core throughput probe (measurement only): blocks workgroups of
// kPeakThreads threads, iters rounds of independent bf16 MFMAs per wave;
// out receives one float per thread.
constexpr int kPeakThreads = 256;
double peak_mfma_flops(int32_t iters, int32_t blocks);
hipError_t launch_peak_mfma(int32_t iters, int32_t blocks, float *out, hipStream_t stream,
                            LaunchEvents ev);
// HBM read probe: blocks workgroups stream the 16-byte units of src;
// out receives one word per thread.
hipError_t launch_peak_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *out,
                            hipStream_t stream, LaunchEvents ev);

// Unshared stage alone for deep chains (p.anc resolved): per query row its
// partial (m, l) into p.tok_ml and unnormalised o into p.tok_o, in the units
// of the staged kernel's online softmax (raw scores, exp2 with scale_log2).
hipError_t launch_token_partials_bf16(const DecodeParams &p, hipStream_t stream,
                                      LaunchEvents ev = {});

// In-place reorder of the Unshared cache: row (t, b) := old row (t, parent[b])
// for t < n_levels, every request and KV head.
struct ReorderParams {
  void *unshared_k;
  void *unshared_v;
  const int32_t *parent;   // [R] rows of BW, stride parent_stride
  int64_t parent_stride;
  int64_t row_bytes;       // D * element size
  int64_t chunk_bytes;     // columns per workgroup (divides row_bytes)
  int32_t R, Hkv, S, BW, n_levels;
};
hipError_t launch_reorder_unshared(const ReorderParams &p, hipStream_t stream,
                                   LaunchEvents ev = {});
int64_t reorder_chunk_bytes(int64_t row_bytes, int32_t BW);

// Valid-path tables and kernels (layout as in xbeam.h).
using TrieLayout = xattn_trie;
constexpr int kMaxTrieLevels = XATTN_TRIE_MAX_LEVELS;
constexpr int kMaxMaskWords = 2048;   // vocabularies up to 65536 tokens

struct MaskParams {
  const uint8_t *table;
  const int32_t *node;     // [R * BW] node id at the masked depth, -1 = dead
  float *logits;           // R * BW rows of V, row stride row_stride
  int64_t row_stride;
  int64_t row_ptr_off, child_tok_off, mask_off;   // sections of the masked depth
  int32_t R, BW, V, words, n_nodes, n_edges;   // nodes at depth d and d + 1
  int32_t dense;           // 1: the depth has dense bit rows
};

struct AdvanceParams {
  const uint8_t *table;
  const int32_t *node;     // [R][BW] nodes at depth d
  const int32_t *parent;   // [R] rows of BW, stride parent_stride
  int64_t parent_stride;
  const int32_t *token;    // [R] rows of BW, stride token_stride
  int64_t token_stride;
  int32_t *new_node;       // [R][BW] nodes at depth d + 1
  int64_t row_ptr_off, child_tok_off;             // sections of depth d
  int32_t R, BW, V, n_nodes, n_edges;             // nodes at depth d and d + 1
};

hipError_t launch_valid_mask(const MaskParams &p, hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_trie_advance(const AdvanceParams &p, hipStream_t stream);
// Host: lay out (and, with host_table, fill) the tables; nullptr or a reason.
const char *build_trie(const int32_t *items, int64_t n_items, int32_t levels, int32_t vocab,
                       int32_t dense_levels, TrieLayout *lay, void *host_table,
                       size_t host_bytes);

// Beam selection: the BW best of BW x V sorted candidates per request.
hipError_t launch_beam_topk(const float *cum, const float *logp, const int32_t *tok, int32_t R,
                            int32_t BW, int32_t V, float *score, int32_t *parent, int32_t *token,
                            int64_t out_stride, hipStream_t stream, LaunchEvents ev = {});
// Candidates per row the beam-selection kernel samples into LDS.
int beam_topk_sample_len(int32_t BW, int32_t V);

// Number of query rows one bf16 workgroup owns for this shape.
int bf16_rows_per_block(const DecodeParams &p);

// Launch geometry of the bf16 staged kernel for p (p.anc, p.step, p.BW,
// p.G, p.M, p.D, p.n_split set): what launch_decode_bf16 would enqueue.
struct Bf16Geometry {
  int rows;            // query rows per workgroup
  int threads;         // per workgroup
  int64_t grid;        // workgroups
  int static_lds;      // bytes of static LDS
  int dyn_lds;         // bytes of dynamic LDS
  int beams_per_block; // most beams one workgroup's rows touch
  bool stage_par;      // parent rows staged in LDS for the in-kernel walk
  bool paired;         // the variant two workgroups of which share a compute unit
};
// LDS one workgroup may use (gfx950: 160 KiB per compute unit).
constexpr int kLdsLimit = 160 * 1024;
Bf16Geometry bf16_geometry(const DecodeParams &p);
// Static LDS bytes per workgroup of the f32 and per-beam kernels.
int f32_lds_bytes(int D);
int per_beam_lds_bytes(int D);
constexpr int kF32Threads = 256;
constexpr int kPerBeamThreads = 256;
// Key splits: combine p.n_split partials (p.part_ml, p.part_o) into p.out.
hipError_t launch_merge_splits_bf16(const DecodeParams &p, hipStream_t stream,
                                    LaunchEvents ev = {});

}  // namespace xattn
