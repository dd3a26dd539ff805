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
// spreads a level's few slices over many workgroups.  A chunk is a whole
// 128-byte cache line of each row where the stage allows it: with narrower
// chunks two workgroups write the two halves of one line, and a partial
// line costs the memory side a merge with the line's old contents (1.3-1.4x
// the time of whole lines at 256 and 512 beams).  Rows whose parent is
// themselves are not rewritten, and a slice whose parents are all the
// identity is not written at all (its rows are read with the parents, in
// the same round trip).
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kThreads = 256;
// Largest stage (BW rows of one column chunk), and the widest chunk.  The
// stage is sized per launch, not to this bound: a workgroup holds only what
// it moves, so more workgroups fit a compute unit's LDS and more rows are in
// flight at once.  Chunks wider than a cache line measured no faster.
constexpr int kStageBytes = 64 * 1024;
constexpr int kChunkMaxBytes = 128;
static_assert(kStageBytes <= kThreads * 16 * 16, "16 units per thread cover the stage");
static_assert(kMaxReorderBeams <= kThreads * 8, "8 parent slots per thread cover the beams");

// UPT: 16-byte units of the stage per thread, PPT: parent slots per thread
// (each the smallest power of two that covers the launch), so every thread
// issues all of its loads before it waits and none of them is redundant.
template <int UPT, int PPT>
__global__ __launch_bounds__(kThreads) void reorder_unshared_kernel(ReorderParams p) {
  // dynamic LDS: the stage (BW rows x chunk_bytes), then BW parent slots
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int moved;
  uint8_t *stage = smem;
  int32_t *par = reinterpret_cast<int32_t *>(smem + (int64_t)p.BW * p.chunk_bytes);

  const int tid = threadIdx.x;
  const int n_cc = (int)(p.row_bytes / p.chunk_bytes);   // column chunks per row
  const int part = blockIdx.x % (2 * n_cc);               // K chunks, then V chunks
  const int slice_id = blockIdx.x / (2 * n_cc);
  const int t = slice_id % p.n_levels;
  const int rk = slice_id / p.n_levels;
  const int k = rk % p.Hkv;
  const int r = rk / p.Hkv;
  const int BW = p.BW;

  const int64_t RB = p.row_bytes;                        // bytes of one row
  const int64_t slice = (((int64_t)r * p.Hkv + k) * p.S + t) * BW * RB;
  const int units_per_row = (int)(p.chunk_bytes / 16);    // 16-byte units per row per chunk
  const int n_units = BW * units_per_row;
  uint8_t *base = static_cast<uint8_t *>(part < n_cc ? p.unshared_k : p.unshared_v) + slice;
  const int64_t c0 = (int64_t)(part % n_cc) * p.chunk_bytes;

  // The parent slots and columns [c0, c0 + chunk) of every row of the slice
  // are loaded together (one memory round trip, not one for the parents and
  // then one for the rows).
  if (tid == 0) moved = 0;
  // this thread's parent slots, loaded into registers first and stored to
  // LDS only after the row loads are issued (indices past BW repeat the
  // last slot and are not stored)
  int32_t pr[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i)
    pr[i] = p.parent[(int64_t)r * p.parent_stride + min(tid + i * kThreads, BW - 1)];
  {
    uint4 v[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = min(tid + i * kThreads, n_units - 1);
      const int b = u / units_per_row, c = u - b * units_per_row;
      v[i] = *reinterpret_cast<const uint4 *>(base + (int64_t)b * RB + c0 + c * 16);
    }
    // (units past the end, in the last round only, repeat the last one: the
    // same bytes to the same place, with no branch to hold the loads apart)
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = min(tid + i * kThreads, n_units - 1);
      *reinterpret_cast<uint4 *>(stage + (int64_t)u * 16) = v[i];
    }
  }
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int b = tid + i * kThreads;
    if (b < BW) {
      const int a = min(max(pr[i], 0), BW - 1);
      par[b] = a;
      mine |= a != b;
    }
  }
  __syncthreads();   // moved = 0 is visible before any thread sets it
  if (mine) moved = 1;   // benign race: every writer stores 1
  __syncthreads();
  if (!moved) return;
  // every read of this chunk is done (the barriers above): write the moved rows
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
  auto pow2_cover = [](int64_t n) {   // smallest of 1, 2, 4, 8, 16 with 256 * it >= n
    int x = 1;
    while (x < 16 && (int64_t)x * kThreads < n) x *= 2;
    return x;
  };
  const int upt = pow2_cover((int64_t)p.BW * (p.chunk_bytes / 16));
  const int ppt = p.BW <= kThreads ? 1 : 8;
  const size_t lds = (size_t)p.BW * (p.chunk_bytes + sizeof(int32_t));
  auto go = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, stream, ev.start,
                            ev.stop, 0u, p);
    else
      hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, stream, p);
  };
  if (ppt == 1) {
    if (upt == 1) go(reorder_unshared_kernel<1, 1>);
    else if (upt == 2) go(reorder_unshared_kernel<2, 1>);
    else if (upt == 4) go(reorder_unshared_kernel<4, 1>);
    else if (upt == 8) go(reorder_unshared_kernel<8, 1>);
    else go(reorder_unshared_kernel<16, 1>);
  } else {
    if (upt == 1) go(reorder_unshared_kernel<1, 8>);
    else if (upt == 2) go(reorder_unshared_kernel<2, 8>);
    else if (upt == 4) go(reorder_unshared_kernel<4, 8>);
    else if (upt == 8) go(reorder_unshared_kernel<8, 8>);
    else go(reorder_unshared_kernel<16, 8>);
  }
  return hipGetLastError();
}

int64_t reorder_chunk_bytes(int64_t row_bytes, int32_t BW) {
  // the largest power-of-two divisor of the row that lets BW rows fit the
  // stage, and at most one cache line: more, smaller workgroups per slice
  int64_t c = row_bytes;
  while (c > 16 && ((int64_t)BW * c > kStageBytes || c > kChunkMaxBytes)) c /= 2;
  return c;
}

}  // namespace xattn
