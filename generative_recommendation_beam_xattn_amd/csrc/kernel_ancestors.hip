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
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsInts = 8192;               // per buffer: 32 KiB of parent rows
constexpr int kPerThread = kLdsInts / kThreads;

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

}  // namespace

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
