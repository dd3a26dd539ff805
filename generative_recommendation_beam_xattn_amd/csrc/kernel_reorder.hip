// In-place reorder of the Unshared cache after beam selection (xGR summary,
// section 2.1, "in-place updates": the generated-token blocks are updated in
// place with direct indices, avoiding write-before-read hazards).
//
// After a step's selection, new beam b descends from slot parent[b].  The
// reorder makes slot b hold beam b's own history: for every level t below
// n_levels and every KV head, row (t, b) takes the old row (t, parent[b]).
// Attention can then use identity parents instead of following chains.
//
// Hazards.  A row may be the source of several beams and the destination of
// another, so rows cannot be moved one by one.  One workgroup owns one
// column chunk of K or of V of one (request, KV head, level) slice -- that
// chunk of all BW rows -- and stages it whole in LDS before writing any of
// it: all reads precede all writes, behind a barrier, and no other
// workgroup touches those bytes.  Splitting the slice by K/V and columns
// spreads a level's few slices over many workgroups.  Rows whose parent is
// themselves are not rewritten, and a slice whose parents are all the
// identity is left untouched without a read.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kThreads = 256;
constexpr int kStageBytes = 32 * 1024;

__global__ __launch_bounds__(kThreads) void reorder_unshared_kernel(ReorderParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStageBytes];
  __shared__ int moved;
  extern __shared__ int32_t par[];   // BW parent slots (dynamic)

  const int tid = threadIdx.x;
  const int n_cc = (int)(p.row_bytes / p.chunk_bytes);   // column chunks per row
  const int part = blockIdx.x % (2 * n_cc);               // K chunks, then V chunks
  const int slice_id = blockIdx.x / (2 * n_cc);
  const int t = slice_id % p.n_levels;
  const int rk = slice_id / p.n_levels;
  const int k = rk % p.Hkv;
  const int r = rk / p.Hkv;
  const int BW = p.BW;

  if (tid == 0) moved = 0;
  __syncthreads();
  int mine = 0;
  for (int b = tid; b < BW; b += kThreads) {
    const int a = min(max(p.parent[(int64_t)r * p.parent_stride + b], 0), BW - 1);
    par[b] = a;
    mine |= a != b;
  }
  if (mine) moved = 1;   // benign race: every writer stores 1
  __syncthreads();
  if (!moved) return;

  const int64_t RB = p.row_bytes;                        // bytes of one row
  const int64_t slice = (((int64_t)r * p.Hkv + k) * p.S + t) * BW * RB;
  const int units_per_row = (int)(p.chunk_bytes / 16);    // 16-byte units per row per chunk
  const int n_units = BW * units_per_row;
  uint8_t *base = static_cast<uint8_t *>(part < n_cc ? p.unshared_k : p.unshared_v) + slice;
  const int64_t c0 = (int64_t)(part % n_cc) * p.chunk_bytes;
  // stage columns [c0, c0 + chunk) of every row of the slice
  for (int u = tid; u < n_units; u += kThreads) {
    const int b = u / units_per_row, c = u - b * units_per_row;
    *reinterpret_cast<uint4 *>(stage + (int64_t)u * 16) =
        *reinterpret_cast<const uint4 *>(base + (int64_t)b * RB + c0 + c * 16);
  }
  __syncthreads();
  // every read of this chunk is done: write the moved rows
  for (int u = tid; u < n_units; u += kThreads) {
    const int b = u / units_per_row, c = u - b * units_per_row;
    const int a = par[b];
    if (a != b)
      *reinterpret_cast<uint4 *>(base + (int64_t)b * RB + c0 + c * 16) =
          *reinterpret_cast<const uint4 *>(stage + ((int64_t)a * units_per_row + c) * 16);
  }
}

}  // namespace

hipError_t launch_reorder_unshared(const ReorderParams &p, hipStream_t stream, LaunchEvents ev) {
  if (p.chunk_bytes <= 0) return hipErrorInvalidConfiguration;
  // per slice: K and V, each in row_bytes / chunk_bytes column chunks
  const int64_t grid = (int64_t)p.R * p.Hkv * p.n_levels * 2 * (p.row_bytes / p.chunk_bytes);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff || p.BW > kMaxReorderBeams || p.chunk_bytes <= 0 ||
      (int64_t)p.BW * p.chunk_bytes > kStageBytes || p.chunk_bytes % 16 != 0 ||
      p.row_bytes % p.chunk_bytes != 0)
    return hipErrorInvalidConfiguration;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(reorder_unshared_kernel, dim3((unsigned)grid), dim3(kThreads),
                          (size_t)p.BW * sizeof(int32_t), stream, ev.start, ev.stop, 0u, p);
  else
    hipLaunchKernelGGL(reorder_unshared_kernel, dim3((unsigned)grid), dim3(kThreads),
                       (size_t)p.BW * sizeof(int32_t), stream, p);
  return hipGetLastError();
}

int64_t reorder_chunk_bytes(int64_t row_bytes, int32_t BW) {
  // the largest power-of-two divisor of the row that lets BW rows fit LDS,
  // and at most 64 bytes: more, smaller workgroups per slice
  int64_t c = row_bytes;
  while (c > 16 && ((int64_t)BW * c > kStageBytes || c > 64)) c /= 2;
  return c;
}

}  // namespace xattn
