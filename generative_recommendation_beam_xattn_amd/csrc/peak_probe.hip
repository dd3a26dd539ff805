// Throughput probes, for measurement only.  The attention kernels'
// fractions are quoted against published peaks, which assume the chip's
// top clock and an ideal memory system.  peak_mfma_kernel keeps every
// SIMD's matrix core busy with independent v_mfma_f32_32x32x16_bf16 chains;
// peak_read_kernel streams a buffer from HBM with 16-byte non-temporal
// loads, four in flight per lane.  Their rates are what this chip delivers
// under such loads.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;   // independent accumulators per wave

__global__ __launch_bounds__(kPeakThreads) void peak_mfma_kernel(float *out, int iters) {
  const int tid = blockIdx.x * kPeakThreads + threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * ((tid + e) & 7));
    b[e] = (__bf16)(0.002f * ((3 * tid + e) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[tid] = s;   // keeps the products live
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kPeakThreads) void peak_read_kernel(const u32x4 *src, int64_t n16,
                                                                 uint32_t *out) {
  const int64_t tid = (int64_t)blockIdx.x * kPeakThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kPeakThreads;
  uint32_t x = 0;
  int64_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^
         d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[tid] = x;   // keeps the loads live
}

}  // namespace

hipError_t launch_peak_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *out,
                            hipStream_t stream, LaunchEvents ev) {
  const u32x4 *s = static_cast<const u32x4 *>(src);
  const int64_t n16 = bytes / 16;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(peak_read_kernel, dim3((unsigned)blocks), dim3(kPeakThreads), 0u,
                          stream, ev.start, ev.stop, 0u, s, n16, out);
  else
    hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)blocks), dim3(kPeakThreads), 0, stream,
                       s, n16, out);
  return hipGetLastError();
}

double peak_mfma_flops(int32_t iters, int32_t blocks) {
  return (double)blocks * (kPeakThreads / 64) * iters * kChains * (2.0 * 32 * 32 * 16);
}

hipError_t launch_peak_mfma(int32_t iters, int32_t blocks, float *out, hipStream_t stream,
                            LaunchEvents ev) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(kPeakThreads), 0u,
                          stream, ev.start, ev.stop, 0u, out, (int)iters);
  else
    hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(kPeakThreads), 0, stream,
                       out, (int)iters);
  return hipGetLastError();
}

}  // namespace xattn
