// Ancestor slots of every beam along the per-step parent indices.
//
// The xGR technical summary (gist.science, paper 2512.11529), section 2.1,
// keeps generated tokens per token and never copies them when beams branch;
// a beam therefore reaches its token at level t by following parent slots
// back from its current slot:  a_s = b,  a_{t-1} = parent_idx[r][t][a_t].
//
// One thread follows one beam.  Parent rows are streamed through LDS a chunk
// of levels at a time, double-buffered: while the threads walk one chunk
// (each step a dependent LDS read rather than a dependent global-memory
// round trip), the next chunk's rows are already being loaded -- into
// registers, every load of the chunk in flight at once -- and stored to
// the other buffer after the walk.
//
// Long chains split the levels into segments walked side by side.  A first
// kernel composes each segment's parent maps: for every slot x at the
// segment's top level, the slot reached at the level below its bottom.  A
// second kernel gives each segment the entry slot of every beam -- the
// beam's slot pushed through the composed maps of the segments above --
// and walks the segment from there, writing the ancestor slots.  The
// dependent chain per beam shrinks from one step per level to one per
// level of a segment plus one per segment.
#include <hip/hip_ext.h>

#include <algorithm>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsInts = 8192;               // per buffer: 32 KiB of parent rows
constexpr int kPerThread = kLdsInts / kThreads;
constexpr int kSegMapInts = 16384;           // composed maps of the segments above: 64 KiB

template <bool kStaged>
__global__ __launch_bounds__(kThreads) void resolve_ancestors_kernel(
    const int32_t *__restrict__ parent_idx, int32_t BW, int32_t S, int32_t step,
    int32_t *__restrict__ anc, AncLayout lay, int32_t blocks_per_request,
    int32_t levels_per_chunk) {
  __shared__ int32_t rows[kStaged ? 2 : 1][kStaged ? kLdsInts : 1];
  const int r = blockIdx.x / blocks_per_request;
  const int b = (blockIdx.x % blocks_per_request) * kThreads + threadIdx.x;
  const bool active = b < BW;
  int32_t *dst = anc + r * lay.stride_r + (int64_t)(active ? b : 0) * lay.stride_b;
  const int32_t *par = parent_idx + (int64_t)r * S * BW;
  int a = active ? b : 0;
  if (active) dst[(int64_t)step * lay.stride_t] = a;
  if constexpr (kStaged) {
    // chunk c covers levels hi(c) = step - c * lpc down to lo(c) = max(1, hi - lpc + 1)
    const int lpc = levels_per_chunk;
    const int n_chunks = step >= 1 ? (step + lpc - 1) / lpc : 0;
    int32_t v[kPerThread];
    auto load = [&](int c) {   // chunk c's rows into registers (rows lo..hi, whole)
      const int hi = step - c * lpc, lo = max(1, hi - lpc + 1);
      const int n = (hi - lo + 1) * BW;
#pragma unroll
      for (int u = 0; u < kPerThread; ++u) {
        const int i = threadIdx.x + u * kThreads;
        v[u] = i < n ? par[(int64_t)lo * BW + i] : 0;
      }
    };
    auto store = [&](int buf) {
#pragma unroll
      for (int u = 0; u < kPerThread; ++u) rows[buf][threadIdx.x + u * kThreads] = v[u];
    };
    if (n_chunks > 0) {
      load(0);
      store(0);
    }
    for (int c = 0; c < n_chunks; ++c) {
      __syncthreads();   // chunk c is in rows[c & 1]; chunk c - 1's buffer is free
      if (c + 1 < n_chunks) load(c + 1);
      const int hi = step - c * lpc, lo = max(1, hi - lpc + 1);
      if (active) {
        const int32_t *rc = rows[c & 1];
        for (int t = hi; t >= lo; --t) {
          a = min(max(rc[(t - lo) * BW + a], 0), BW - 1);
          dst[(int64_t)(t - 1) * lay.stride_t] = a;
        }
      }
      if (c + 1 < n_chunks) store((c + 1) & 1);
    }
  } else {
    // a single parent row does not fit the LDS budget: walk global memory
    if (active) {
      for (int t = step; t >= 1; --t) {
        a = min(max(par[(int64_t)t * BW + a], 0), BW - 1);
        dst[(int64_t)(t - 1) * lay.stride_t] = a;
      }
    }
  }
}

// n consecutive int32 from global memory into LDS, eight loads per thread
// in flight at a time.
__device__ inline void copy_to_lds(const int32_t *src, int n, int32_t *dst) {
  constexpr int kBatch = 8;
  for (int base = 0; base < n; base += kBatch * kThreads) {
    int32_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * kThreads + threadIdx.x;
      v[u] = i < n ? src[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * kThreads + threadIdx.x;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Segment j covers parent levels hi_j = step - j * lps down to
// lo_j = max(1, hi_j - lps + 1); its rows are staged in LDS ascending.
__device__ inline void segment_rows(const int32_t *par, int32_t BW, int hi, int lo,
                                    int32_t *rows) {
  copy_to_lds(par + (int64_t)lo * BW, (hi - lo + 1) * BW, rows);
}

// LDS of both segment kernels (dynamic, sized to the shape): the segment's
// parent rows, lps * BW int32, then (walk) the composed maps of the
// segments above, up to (n_seg - 1) * BW int32.
__global__ __launch_bounds__(kThreads) void ancestor_segments_kernel(
    const int32_t *__restrict__ parent_idx, int32_t BW, int32_t S, int32_t step, int32_t lps,
    int32_t n_seg, int32_t *__restrict__ fmap) {
  extern __shared__ int32_t seg_lds[];
  int32_t *rows = seg_lds;
  const int r = blockIdx.x / n_seg, j = blockIdx.x % n_seg;
  const int hi = step - j * lps, lo = max(1, hi - lps + 1);
  segment_rows(parent_idx + (int64_t)r * S * BW, BW, hi, lo, rows);
  __syncthreads();
  int32_t *f = fmap + ((int64_t)r * n_seg + j) * BW;
  for (int x = threadIdx.x; x < BW; x += kThreads) {
    int a = x;
    for (int t = hi; t >= lo; --t) a = min(max(rows[(t - lo) * BW + a], 0), BW - 1);
    f[x] = a;
  }
}

__global__ __launch_bounds__(kThreads) void ancestor_segment_walk_kernel(
    const int32_t *__restrict__ parent_idx, int32_t BW, int32_t S, int32_t step, int32_t lps,
    int32_t n_seg, const int32_t *__restrict__ fmap, int32_t *__restrict__ anc, AncLayout lay) {
  extern __shared__ int32_t seg_lds[];
  int32_t *rows = seg_lds, *maps = seg_lds + lps * BW;
  const int r = blockIdx.x / n_seg, j = blockIdx.x % n_seg;
  const int hi = step - j * lps, lo = max(1, hi - lps + 1);
  segment_rows(parent_idx + (int64_t)r * S * BW, BW, hi, lo, rows);
  copy_to_lds(fmap + (int64_t)r * n_seg * BW, j * BW, maps);
  __syncthreads();
  for (int b = threadIdx.x; b < BW; b += kThreads) {
    int32_t *dst = anc + r * lay.stride_r + (int64_t)b * lay.stride_b;
    int a = b;
    for (int i = 0; i < j; ++i) a = maps[i * BW + a];   // the beam's slot at level hi
    if (j == 0) dst[(int64_t)step * lay.stride_t] = a;
    for (int t = hi; t >= lo; --t) {
      a = min(max(rows[(t - lo) * BW + a], 0), BW - 1);
      dst[(int64_t)(t - 1) * lay.stride_t] = a;
    }
  }
}

}  // namespace

int ancestor_segment_levels(int32_t BW, int32_t step) {
  if (BW < 1 || step < 1 || BW > kLdsInts / 8) return 0;
  const int lps = std::min(64, kLdsInts / BW);
  const int64_t n_seg = (step + lps - 1) / lps;
  if (n_seg < 2 || n_seg * BW > kSegMapInts) return 0;
  return lps;
}

hipError_t launch_resolve_ancestors_segmented(const int32_t *parent_idx, int32_t R, int32_t BW,
                                              int32_t S, int32_t step, int32_t *anc,
                                              AncLayout layout, int32_t *fmap,
                                              hipStream_t stream, LaunchEvents ev) {
  const int lps = ancestor_segment_levels(BW, step);
  if (lps == 0) return hipErrorInvalidValue;
  const int32_t n_seg = (step + lps - 1) / lps;
  const int64_t grid = (int64_t)R * n_seg;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const uint32_t lds_rows = (uint32_t)(lps * BW) * sizeof(int32_t);
  const uint32_t lds_walk = lds_rows + (uint32_t)((n_seg - 1) * BW) * sizeof(int32_t);
  if (ev.start)
    hipExtLaunchKernelGGL(ancestor_segments_kernel, dim3((unsigned)grid), dim3(kThreads), lds_rows,
                          stream, ev.start, nullptr, 0u, parent_idx, BW, S, step, lps, n_seg,
                          fmap);
  else
    hipLaunchKernelGGL(ancestor_segments_kernel, dim3((unsigned)grid), dim3(kThreads), lds_rows,
                       stream, parent_idx, BW, S, step, lps, n_seg, fmap);
  if (ev.stop)
    hipExtLaunchKernelGGL(ancestor_segment_walk_kernel, dim3((unsigned)grid), dim3(kThreads),
                          lds_walk, stream, nullptr, ev.stop, 0u, parent_idx, BW, S, step, lps,
                          n_seg, fmap, anc, layout);
  else
    hipLaunchKernelGGL(ancestor_segment_walk_kernel, dim3((unsigned)grid), dim3(kThreads),
                       lds_walk, stream, parent_idx, BW, S, step, lps, n_seg, fmap, anc, layout);
  return hipGetLastError();
}

hipError_t launch_resolve_ancestors(const int32_t *parent_idx, int32_t R, int32_t BW, int32_t S,
                                    int32_t step, int32_t *anc, AncLayout layout,
                                    hipStream_t stream, LaunchEvents ev) {
  const int32_t bpr = (BW + kThreads - 1) / kThreads;
  const int64_t grid = (int64_t)R * bpr;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool lds = BW <= kLdsInts;
  const int32_t chunk = lds ? max(1, min(step, kLdsInts / BW)) : 1;
  auto kernel = lds ? resolve_ancestors_kernel<true> : resolve_ancestors_kernel<false>;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0u, stream, ev.start,
                          ev.stop, 0u, parent_idx, BW, S, step, anc, layout, bpr, chunk);
  else
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, parent_idx, BW,
                       S, step, anc, layout, bpr, chunk);
  return hipGetLastError();
}

}  // namespace xattn
