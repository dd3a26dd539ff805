// Ancestor slots of every beam along the per-step parent indices.
//
// The xGR technical summary (gist.science, paper 2512.11529), section 2.1,
// keeps generated tokens per token and never copies them when beams branch;
// a beam therefore reaches its token at level t by following parent slots
// back from its current slot:  a_s = b,  a_{t-1} = parent_idx[r][t][a_t].
//
// One thread follows one beam.  Parent rows are staged through LDS a chunk
// of levels at a time with coalesced loads, so each step of the walk is a
// dependent LDS read rather than a dependent global-memory round trip.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsInts = 8192;  // 32 KiB of staged parent rows

template <bool kStaged>
__global__ __launch_bounds__(kThreads) void resolve_ancestors_kernel(
    const int32_t *__restrict__ parent_idx, int32_t BW, int32_t S, int32_t step,
    int32_t *__restrict__ anc, AncLayout lay, int32_t blocks_per_request,
    int32_t levels_per_chunk) {
  __shared__ int32_t rows[kStaged ? kLdsInts : 1];
  const int r = blockIdx.x / blocks_per_request;
  const int b = (blockIdx.x % blocks_per_request) * kThreads + threadIdx.x;
  const bool active = b < BW;
  int32_t *dst = anc + r * lay.stride_r + (int64_t)(active ? b : 0) * lay.stride_b;
  const int32_t *par = parent_idx + (int64_t)r * S * BW;
  int a = active ? b : 0;
  if (active) dst[(int64_t)step * lay.stride_t] = a;
  if constexpr (kStaged) {
    for (int hi = step; hi >= 1; hi -= levels_per_chunk) {
      const int lo = max(1, hi - levels_per_chunk + 1);
      const int n = (hi - lo + 1) * BW;
      __syncthreads();  // the previous chunk has been consumed
      for (int i = threadIdx.x; i < n; i += kThreads) rows[i] = par[(int64_t)lo * BW + i];
      __syncthreads();
      if (active) {
        for (int t = hi; t >= lo; --t) {
          a = min(max(rows[(t - lo) * BW + a], 0), BW - 1);
          dst[(int64_t)(t - 1) * lay.stride_t] = a;
        }
      }
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
