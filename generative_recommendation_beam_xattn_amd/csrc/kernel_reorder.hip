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
// chunk of all BW rows -- and gathers, for every row that moves, its
// parent's chunk into registers; every wave waits for all of its loads and
// the workgroup synchronises before any thread writes.  All reads of the
// chunk thus precede all writes, and no other workgroup touches those
// bytes.  Rows whose parent is themselves are not written; a row is read
// once per beam it is the parent of, the repeats from the caches.
// Splitting the slice by K/V and columns spreads a level's few slices over
// many workgroups.  A chunk is a whole 128-byte cache line of each row where
// the registers allow it: with narrower chunks two workgroups write the two
// halves of one line, and a partial line costs the memory side a merge with
// the line's old contents (1.3-1.4x the time of whole lines at 256 and 512
// beams).  Keeping the chunk in registers rather than staging it in LDS
// leaves a compute unit's workgroup count to its waves, not to its LDS.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

// (a native vector type: the HIP uint4 struct kept across the barrier is
// not split into registers and goes to scratch)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// Largest column chunk of a slice a workgroup holds in registers (BW rows x
// chunk bytes, at most 16 units of 16 bytes per thread), and the widest
// chunk: a cache line (wider chunks measured no faster).
constexpr int kChunkLimitBytes = 64 * 1024;
constexpr int kChunkMaxBytes = 128;
static_assert(kChunkLimitBytes <= kThreads * 16 * 16, "16 units per thread cover the chunk");
static_assert(kMaxReorderBeams <= kThreads * 8, "8 parent slots per thread cover the beams");

// UPT: 16-byte units of the chunk per thread, the smallest power of two that
// covers the launch.
template <int UPT>
__global__ __launch_bounds__(kThreads) void reorder_unshared_kernel(ReorderParams p) {
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

  const int64_t RB = p.row_bytes;                        // bytes of one row
  const int64_t slice = (((int64_t)r * p.Hkv + k) * p.S + t) * BW * RB;
  const int units_per_row = (int)(p.chunk_bytes / 16);    // 16-byte units per row per chunk
  const int n_units = BW * units_per_row;
  uint8_t *base = static_cast<uint8_t *>(part < n_cc ? p.unshared_k : p.unshared_v) + slice;
  const int64_t c0 = (int64_t)(part % n_cc) * p.chunk_bytes;

  {
    // the parent slots, all of the thread's loads in flight together
    int32_t pv[kMaxReorderBeams / kThreads];
#pragma unroll
    for (int j = 0; j < kMaxReorderBeams / kThreads; ++j) {
      const int b = tid + j * kThreads;
      if (b < BW) pv[j] = p.parent[(int64_t)r * p.parent_stride + b];
    }
#pragma unroll
    for (int j = 0; j < kMaxReorderBeams / kThreads; ++j) {
      const int b = tid + j * kThreads;
      if (b < BW) par[b] = min(max(pv[j], 0), BW - 1);
    }
  }
  __syncthreads();
  // each unit of a moved row takes the same unit of its parent's row,
  // gathered into registers (every unit loads, with no branch to hold the
  // loads apart; units past the end repeat the last one); only moved rows
  // are written
  u32x4 v[UPT];
  uint32_t mv = 0;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = min(tid + i * kThreads, n_units - 1);
    const int b = u / units_per_row, c = u - b * units_per_row;
    const int a = par[b];
    v[i] = *reinterpret_cast<const u32x4 *>(base + (int64_t)a * RB + c0 + c * 16);
    mv |= (uint32_t)(a != b && tid + i * kThreads < n_units) << i;
  }
  // A row may be one beam's source and another's destination: every load of
  // the workgroup has returned (vmcnt 0 in each wave, then the barrier)
  // before any thread writes.  s_waitcnt immediate (gfx9 encoding): vmcnt 0
  // in bits 3:0 and 15:14, expcnt left at 7 in bits 6:4, lgkmcnt 0 in 11:8.
  __builtin_amdgcn_s_waitcnt(0x70);
  __syncthreads();
  // (written once: past the caches)
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    if ((mv >> i) & 1u) {
      const int u = tid + i * kThreads;
      const int b = u / units_per_row, c = u - b * units_per_row;
      __builtin_nontemporal_store(v[i],
                                  reinterpret_cast<u32x4 *>(base + (int64_t)b * RB + c0 + c * 16));
    }
  }
}

}  // namespace

hipError_t launch_reorder_unshared(const ReorderParams &p, hipStream_t stream, LaunchEvents ev) {
  if (p.chunk_bytes <= 0) return hipErrorInvalidConfiguration;
  // per slice: K and V, each in row_bytes / chunk_bytes column chunks
  const int64_t grid = (int64_t)p.R * p.Hkv * p.n_levels * 2 * (p.row_bytes / p.chunk_bytes);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff || p.BW > kMaxReorderBeams || p.chunk_bytes <= 0 ||
      (int64_t)p.BW * p.chunk_bytes > kChunkLimitBytes || p.chunk_bytes % 16 != 0 ||
      p.row_bytes % p.chunk_bytes != 0)
    return hipErrorInvalidConfiguration;
  auto pow2_cover = [](int64_t n) {   // smallest of 1, 2, 4, 8, 16 with 256 * it >= n
    int x = 1;
    while (x < 16 && (int64_t)x * kThreads < n) x *= 2;
    return x;
  };
  const int upt = pow2_cover((int64_t)p.BW * (p.chunk_bytes / 16));
  const size_t lds = (size_t)p.BW * sizeof(int32_t);
  auto go = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, stream, ev.start,
                            ev.stop, 0u, p);
    else
      hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, stream, p);
  };
  if (upt == 1) go(reorder_unshared_kernel<1>);
  else if (upt == 2) go(reorder_unshared_kernel<2>);
  else if (upt == 4) go(reorder_unshared_kernel<4>);
  else if (upt == 8) go(reorder_unshared_kernel<8>);
  else go(reorder_unshared_kernel<16>);
  return hipGetLastError();
}

int64_t reorder_chunk_bytes(int64_t row_bytes, int32_t BW) {
  // the largest power-of-two divisor of the row that lets BW rows fit a
  // workgroup's registers, and at most one cache line: more, smaller
  // workgroups per slice
  int64_t c = row_bytes;
  while (c > 16 && ((int64_t)BW * c > kChunkLimitBytes || c > kChunkMaxBytes)) c /= 2;
  return c;
}

}  // namespace xattn
