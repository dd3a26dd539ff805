// Staged decode attention in float32 (fp32 inputs, fp32 arithmetic).
//
// Same operation as the bf16 kernel -- the xAttention stages of the xGR
// technical summary (gist.science, paper 2512.11529), section 2.1 -- for
// float32 caches, where results must stay within fp32 rounding of the exact
// answer.  The matrix cores' bf16 path would not meet that, so this kernel
// runs on the vector ALUs.
//
// One workgroup (4 waves) owns one query row (r, b, h).  Wave w takes every
// fourth key of each stage; a lane owns D/64 dimensions, scores are
// wave-reduced, and each wave keeps an online-softmax state per stage.  The
// four waves' states are merged per stage in LDS, then the Shared and
// Unshared partials are merged with the OnlineSoftmax combine.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kWaves = 4;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int D>
struct StageState {
  static constexpr int DL = D / 64;
  float m = -INFINITY, l = 0.f, o[DL];
  __device__ StageState() {
#pragma unroll
    for (int i = 0; i < DL; ++i) o[i] = 0.f;
  }
  // one more key with raw score sc (dot units) and value row v
  __device__ void add(float sc, const float *v, int lane, float c) {
    const float mn = fmaxf(m, sc);
    const float alpha = __builtin_amdgcn_exp2f((m - mn) * c);
    const float pr = __builtin_amdgcn_exp2f((sc - mn) * c);
    l = l * alpha + pr;
    m = mn;
#pragma unroll
    for (int i = 0; i < DL; ++i) o[i] = fmaf(o[i], alpha, pr * v[lane + 64 * i]);
  }
};

static_assert(kWaves * 64 == kF32Threads, "threads per workgroup");

// Static LDS: the walked ancestor slots, and per stage and wave (m, l, o).
template <int D>
struct F32Lds {
  int32_t anc_s[kMaxInKernelLevels];
  float red_m[2][kWaves], red_l[2][kWaves];
  float red_o[2][kWaves][D];
};

template <int D>
__global__ __launch_bounds__(kWaves * 64) void decode_f32_kernel(DecodeParams p) {
  constexpr int DL = D / 64;
  __shared__ F32Lds<D> lds;
  int32_t *anc_s = lds.anc_s;
  float (*red_m)[kWaves] = lds.red_m;
  float (*red_l)[kWaves] = lds.red_l;
  float (*red_o)[kWaves][D] = lds.red_o;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;  // (r, b, h) in row-major order
  const int h = (int)(row % p.Hq);
  const int b = (int)((row / p.Hq) % p.BW);
  const int r = (int)(row / ((int64_t)p.Hq * p.BW));
  const int k = h / p.G;
  const int BW = p.BW, step = p.step;
  const int L = min(max(p.prompt_len[r], 0), p.Lmax);
  const float c = p.scale_log2;

  if (p.anc == nullptr && threadIdx.x == 0) {
    const int32_t *par = p.parent_idx + (int64_t)r * p.S * BW;
    int a = b;
    anc_s[step] = a;
    for (int t = step; t >= 1; --t) {
      a = min(max(par[(int64_t)t * BW + a], 0), BW - 1);
      anc_s[t - 1] = a;
    }
  }
  __syncthreads();
  // the slots walked, when asked for: anc_out [R][step + 1][BW], written by
  // the beam's first query row
  if (p.anc == nullptr && p.anc_out && h == 0)
    for (int t = threadIdx.x; t <= step; t += kWaves * 64)
      p.anc_out[((int64_t)r * (step + 1) + t) * BW + b] = anc_s[t];

  const float *qp = static_cast<const float *>(p.q) + row * D;
  float qv[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) qv[i] = qp[lane + 64 * i];

  // Shared stage: prompt rows j = wave, wave + 4, ...
  StageState<D> st[2];
  const float *sk = static_cast<const float *>(p.shared_k) + ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const float *sv = static_cast<const float *>(p.shared_v) + ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  for (int j = wave; j < L; j += kWaves) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) part = fmaf(qv[i], sk[(int64_t)j * D + lane + 64 * i], part);
    st[0].add(wave_sum(part), sv + (int64_t)j * D, lane, c);
  }
  // Unshared stage: the beam's ancestor token at levels t = wave, wave + 4, ...
  const int64_t ubase = ((int64_t)r * p.Hkv + k) * p.S * BW;
  const float *uk = static_cast<const float *>(p.unshared_k);
  const float *uv = static_cast<const float *>(p.unshared_v);
  for (int t = wave; t <= step; t += kWaves) {
    const int slot = p.anc ? min(max(p.anc[((int64_t)r * (step + 1) + t) * BW + b], 0), BW - 1)
                           : anc_s[t];
    const int64_t off = (ubase + (int64_t)t * BW + slot) * D;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) part = fmaf(qv[i], uk[off + lane + 64 * i], part);
    st[1].add(wave_sum(part), uv + off, lane, c);
  }

  // merge the four waves of each stage
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (lane == 0) {
      red_m[s][wave] = st[s].m;
      red_l[s][wave] = st[s].l;
    }
#pragma unroll
    for (int i = 0; i < DL; ++i) red_o[s][wave][lane + 64 * i] = st[s].o[i];
  }
  __syncthreads();
  if (wave != 0) return;

  float sm[2], sl[2], so[2][DL];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_m[s][w]);
    float ll = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) so[s][i] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (red_l[s][w] > 0.f) {
        const float f = __builtin_amdgcn_exp2f((red_m[s][w] - mm) * c);
        ll = fmaf(red_l[s][w], f, ll);
#pragma unroll
        for (int i = 0; i < DL; ++i) so[s][i] = fmaf(red_o[s][w][lane + 64 * i], f, so[s][i]);
      }
    }
    sm[s] = mm;
    sl[s] = ll;
  }

  // OnlineSoftmax merge of the Shared (0) and Unshared (1) partials
  const float mm = fmaxf(sm[0], sm[1]);
  const float w0 = sl[0] > 0.f ? __builtin_amdgcn_exp2f((sm[0] - mm) * c) : 0.f;
  const float w1 = __builtin_amdgcn_exp2f((sm[1] - mm) * c);
  const float z = sl[0] * w0 + sl[1] * w1;
  float *op = static_cast<float *>(p.out) + row * D;
#pragma unroll
  for (int i = 0; i < DL; ++i) op[lane + 64 * i] = (so[0][i] * w0 + so[1][i] * w1) / z;

  if (p.lse && lane == 0) p.lse[row] = mm * p.scale + __logf(z);
  const int64_t n_rows_all = (int64_t)p.R * BW * p.Hq;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int64_t ri = s * n_rows_all + row;
    if (p.stage_ml && lane == 0) {
      p.stage_ml[ri * 2 + 0] = sl[s] > 0.f ? sm[s] * p.scale : -INFINITY;
      p.stage_ml[ri * 2 + 1] = sl[s];
    }
    if (p.stage_o) {
#pragma unroll
      for (int i = 0; i < DL; ++i)
        p.stage_o[ri * D + lane + 64 * i] = sl[s] > 0.f ? so[s][i] / sl[s] : 0.f;
    }
  }
}

}  // namespace

namespace {

template <int D>
void launch_f32_d(const DecodeParams &p, unsigned grid, hipStream_t stream, LaunchEvents ev) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(decode_f32_kernel<D>, dim3(grid), dim3(kWaves * 64), 0u, stream,
                          ev.start, ev.stop, 0u, p);
  else
    hipLaunchKernelGGL(decode_f32_kernel<D>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
}

}  // namespace

int f32_lds_bytes(int D) { return D == 64 ? (int)sizeof(F32Lds<64>) : (int)sizeof(F32Lds<128>); }

hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t stream, LaunchEvents ev) {
  const int64_t grid = (int64_t)p.R * p.BW * p.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (p.D == 64)
    launch_f32_d<64>(p, (unsigned)grid, stream, ev);
  else if (p.D == 128)
    launch_f32_d<128>(p, (unsigned)grid, stream, ev);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace xattn
