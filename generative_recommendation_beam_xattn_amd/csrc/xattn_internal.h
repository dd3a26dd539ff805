// Internal declarations of libxattn.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

// Chains of at most this many levels are walked inside the attention kernel
// (slots kept in LDS); deeper chains are resolved by the ancestor kernel into
// the workspace first.
constexpr int kMaxInKernelLevels = 16;

// Largest beam width the beam-selection kernel takes.
constexpr int kMaxTopkBeams = 512;
// Largest beam width the Unshared-cache reorder takes.
constexpr int kMaxReorderBeams = 2048;

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
  float *lse;          // optional taps (debug entry only)
  float *stage_ml;
  float *stage_o;
  int32_t R, BW, Hq, Hkv, D, Lmax, S, step;
  int32_t G;           // Hq / Hkv, query heads per KV head
  int32_t M;           // BW * G query rows per (request, KV head)
  int32_t n_rb;        // row blocks per (request, KV head)
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e): scores go through exp2
};

// Ancestor output layouts: element (r, b, t) lives at
//   r * stride_r + b * stride_b + t * stride_t.
struct AncLayout {
  int64_t stride_r, stride_b, stride_t;
};

// Optional pair of events bound to one kernel dispatch (hipExtLaunchKernel):
// start and stop then time that kernel alone.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_resolve_ancestors(const int32_t *parent_idx, int32_t R, int32_t BW, int32_t S,
                                    int32_t step, int32_t *anc, AncLayout layout,
                                    hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams &p, bool taps, hipStream_t stream,
                              LaunchEvents ev = {});
hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_decode_per_beam_bf16(const DecodeParams &p, hipStream_t stream,
                                       LaunchEvents ev = {});

// In-place reorder of the Unshared cache: row (t, b) := old row (t, parent[b])
// for t < n_levels, every request and KV head.
struct ReorderParams {
  void *unshared_k;
  void *unshared_v;
  const int32_t *parent;   // [R] rows of BW, stride parent_stride
  int64_t parent_stride;
  int64_t row_bytes;       // D * element size
  int64_t chunk_bytes;     // columns staged per pass (divides row_bytes)
  int32_t R, Hkv, S, BW, n_levels;
};
hipError_t launch_reorder_unshared(const ReorderParams &p, hipStream_t stream,
                                   LaunchEvents ev = {});
int64_t reorder_chunk_bytes(int64_t row_bytes, int32_t BW);

// Beam selection: the BW best of BW x V sorted candidates per request.
hipError_t launch_beam_topk(const float *cum, const float *logp, const int32_t *tok, int32_t R,
                            int32_t BW, int32_t V, float *score, int32_t *parent, int32_t *token,
                            int64_t out_stride, hipStream_t stream, LaunchEvents ev = {});
// Candidates per row the beam-selection kernel samples into LDS.
int beam_topk_sample_len(int32_t BW, int32_t V);

// Number of query rows one bf16 workgroup owns for this shape.
int bf16_rows_per_block(const DecodeParams &p);

}  // namespace xattn
