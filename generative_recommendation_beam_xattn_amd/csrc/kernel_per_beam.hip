// Per-beam decode attention: the comparison baseline the xGR summary
// measures xAttention against (section 1 and section 4: PagedAttention-style
// kernels run every beam as a sequence of its own and re-read the shared
// prompt KV for each beam).
//
// Same operation and result as the staged kernels -- softmax attention of
// each query row over [prompt rows 0..L_r-1 ; the beam's own generated
// token at levels 0..s] -- computed the way a per-sequence decode kernel
// does it: one workgroup per (request r, beam b, KV head k) streams that
// beam's whole sequence, the prompt included, for the G query heads of k.
// Nothing is shared between the beams of a request, so the prompt's K/V
// cross the memory hierarchy once per beam.
//
// A key row (D bf16) is read by LPK = D / 8 lanes, 16 bytes each, so a
// wave reads 64 / LPK rows per load instruction, fully coalesced.  Each
// lane group keeps an online-softmax state per query row for the keys it
// visits (dot products with v_dot2_f32_bf16, reduced over the group); the
// states of all groups of the 4 waves are merged through LDS at the end.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kRowsPerPass = 4;   // query rows a pass keeps state for
constexpr int kAncLds = 2048;     // ancestor slots staged in LDS (levels)
constexpr int kKeysInFlight = 4;  // keys per lane group whose loads go out together

__device__ inline float lo_f(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float hi_f(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// x from another lane of the same 16-lane DPP row, by DPP control `ctrl`.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of LPK (8 or 16) lanes, returned to every lane
// of the group, on the vector ALUs: pairs (quad_perm 1,0,3,2), quads
// (quad_perm 2,3,0,1), half rows (row_half_mirror), rows (row_mirror).
template <int LPK>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(LPK == 8 || LPK == 16, "a lane group is half or all of a DPP row");
  s += dpp_f<0xB1>(s);
  s += dpp_f<0x4E>(s);
  s += dpp_f<0x141>(s);
  if constexpr (LPK == 16) s += dpp_f<0x140>(s);
  return s;
}

// A lane group's running maximum only moves when a score exceeds it by
// more than p.lazy_log2 (8 on the decode path: 2^8) in the exp2 domain;
// until then exp2(s - m) may exceed 1 (by at most 256), which the fp32 sums
// hold without loss of range.

// TOKENS: the Unshared stage alone (keys = the beam's tokens at levels
// 0..step), written as an online-softmax partial for the staged kernel to
// start from, instead of normalised output.
static_assert(kWaves * 64 == kPerBeamThreads, "threads per workgroup");

// Static LDS: the beam's ancestor slots, and each lane group's per-row state.
template <int D>
struct PerBeamLds {
  static constexpr int NSG = kWaves * (64 / (D / 8));   // lane groups
  int32_t anc_s[kAncLds];
  float red_o[NSG][kRowsPerPass][D];
  float red_ml[NSG][kRowsPerPass][2];
};

template <int D, bool TOKENS>
__global__ __launch_bounds__(kWaves * 64) void decode_per_beam_kernel(DecodeParams p) {
  constexpr int LPK = D / 8;        // lanes per key row
  constexpr int KPW = 64 / LPK;     // key rows per wave per load
  constexpr int NSG = kWaves * KPW; // lane groups in the workgroup
  static_assert(NSG == PerBeamLds<D>::NSG, "lane groups");
  __shared__ PerBeamLds<D> lds;
  int32_t *anc_s = lds.anc_s;
  float (*red_o)[kRowsPerPass][D] = lds.red_o;
  float (*red_ml)[kRowsPerPass][2] = lds.red_ml;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPK, part = lane % LPK;
  const int sg = wave * KPW + sub;
  // per-beam comparison: KV head fastest, as a per-sequence grid orders it;
  // the Unshared stage: beam fastest, so workgroups running side by side
  // read neighbouring rows (t, b), (t, b + 1), ... of each level
  const int k = TOKENS ? (blockIdx.x / p.BW) % p.Hkv : blockIdx.x % p.Hkv;
  const int b = TOKENS ? blockIdx.x % p.BW : (blockIdx.x / p.Hkv) % p.BW;
  const int r = blockIdx.x / (p.Hkv * p.BW);
  const int step = p.step, BW = p.BW, G = p.G;
  const float c = p.scale_log2;
  const float thr = p.lazy_log2 / c;   // in raw dot-product units

  // the beam's ancestor slot at every level: walked here for short chains,
  // resolved into the workspace beforehand for deep ones
  if (p.anc == nullptr) {
    if (tid == 0) {
      int a = b;
      anc_s[step] = a;
      const int32_t *par = p.parent_idx + (int64_t)r * p.S * BW;
      for (int t = step; t >= 1; --t) {
        a = min(max(par[(int64_t)t * BW + a], 0), BW - 1);
        anc_s[t - 1] = a;
      }
    }
    __syncthreads();
    // the slots walked, when asked for: anc_out [R][step + 1][BW]
    if (!TOKENS && p.anc_out && k == 0)
      for (int t = tid; t <= step; t += kWaves * 64)
        p.anc_out[((int64_t)r * (step + 1) + t) * BW + b] = anc_s[t];
  }
  // resolved slots (deep chains) are staged in LDS too when they fit, so a
  // token row's address waits on an LDS read, not a global one
  const bool anc_in_lds = p.anc == nullptr || step + 1 <= kAncLds;
  if (p.anc && anc_in_lds) {
    for (int t = tid; t <= step; t += kWaves * 64)
      anc_s[t] = min(max(p.anc[((int64_t)r * (step + 1) + t) * BW + b], 0), BW - 1);
    __syncthreads();
  }
  auto anc_of = [&](int t) {
    return anc_in_lds ? anc_s[t]
                      : min(max(p.anc[((int64_t)r * (step + 1) + t) * BW + b], 0), BW - 1);
  };

  const int L = TOKENS ? 0 : min(max(p.prompt_len[r], 0), p.Lmax);
  const int n_keys = L + step + 1;
  const uint16_t *skg = static_cast<const uint16_t *>(p.shared_k) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *svg = static_cast<const uint16_t *>(p.shared_v) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *ukg = static_cast<const uint16_t *>(p.unshared_k) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  const uint16_t *uvg = static_cast<const uint16_t *>(p.unshared_v) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  const uint16_t *qg = static_cast<const uint16_t *>(p.q);
  uint16_t *og = static_cast<uint16_t *>(p.out);

  for (int h0 = 0; h0 < G; h0 += kRowsPerPass) {
    const int nr = min(kRowsPerPass, G - h0);
    // this lane's 8 dims of each query row of the pass
    uint4 qv[kRowsPerPass];
#pragma unroll
    for (int j = 0; j < kRowsPerPass; ++j) {
      const int hh = k * G + h0 + min(j, nr - 1);
      qv[j] = *reinterpret_cast<const uint4 *>(qg + (((int64_t)r * BW + b) * p.Hq + hh) * D +
                                               part * 8);
    }
    float m[kRowsPerPass], l[kRowsPerPass], o[kRowsPerPass][8];
#pragma unroll
    for (int j = 0; j < kRowsPerPass; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }
    // a lane group's keys sg, sg + NSG, ...: kKeysInFlight of them at a
    // time, their K and V loads all issued before the first is used
    for (int i0 = sg; i0 < n_keys; i0 += NSG * kKeysInFlight) {
      uint4 kvu[kKeysInFlight], vvu[kKeysInFlight];
#pragma unroll
      for (int u = 0; u < kKeysInFlight; ++u) {
        const int i = min(i0 + u * NSG, n_keys - 1);   // past the end: a valid row, unused
        const uint16_t *kr, *vr;
        if (i < L) {
          kr = skg + (int64_t)i * D;
          vr = svg + (int64_t)i * D;
        } else {
          const int t = i - L;
          const int64_t e = ((int64_t)t * BW + anc_of(t)) * D;
          kr = ukg + e;
          vr = uvg + e;
        }
        // each K/V row is read once per workgroup: streamed past the caches
        kvu[u] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kr + part * 8)));
        vvu[u] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vr + part * 8)));
      }
      // scores of the keys in flight against the pass's query rows (a key
      // past the end scores -inf and adds nothing)
      float sc[kKeysInFlight][kRowsPerPass];
#pragma unroll
      for (int u = 0; u < kKeysInFlight; ++u) {
        const uint32_t kw[4] = {kvu[u].x, kvu[u].y, kvu[u].z, kvu[u].w};
#pragma unroll
        for (int j = 0; j < kRowsPerPass; ++j) {
          const uint32_t qw[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w};
          float x = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[e]),
                                                __builtin_bit_cast(bf16x2, kw[e]), x, false);
          x = group_sum<LPK>(x);
          sc[u][j] = i0 + u * NSG < n_keys ? x : -INFINITY;
        }
      }
      // online softmax of this lane group's keys (scores in exp2 units).
      // The maximum is raised lazily and rarely: then the keys are taken
      // one by one with the full update; otherwise they add exp2(s - m).
      bool raise = false;
#pragma unroll
      for (int u = 0; u < kKeysInFlight; ++u)
#pragma unroll
        for (int j = 0; j < kRowsPerPass; ++j) raise |= sc[u][j] > m[j] + thr;
      if (__any(raise)) {
#pragma unroll
        for (int u = 0; u < kKeysInFlight; ++u) {
          const uint32_t vw[4] = {vvu[u].x, vvu[u].y, vvu[u].z, vvu[u].w};
#pragma unroll
          for (int j = 0; j < kRowsPerPass; ++j) {
            const float x = sc[u][j];
            if (x > m[j] + thr) {
              const float mn = fmaxf(m[j], x);
              const float alpha = __builtin_amdgcn_exp2f((m[j] - mn) * c);   // 0 while m is -inf
              m[j] = mn;
              l[j] *= alpha;
#pragma unroll
              for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
            }
            const float pr = __builtin_amdgcn_exp2f((x - m[j]) * c);
            l[j] += pr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[j][2 * e] = fmaf(pr, lo_f(vw[e]), o[j][2 * e]);
              o[j][2 * e + 1] = fmaf(pr, hi_f(vw[e]), o[j][2 * e + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < kKeysInFlight; ++u) {
          const uint32_t vw[4] = {vvu[u].x, vvu[u].y, vvu[u].z, vvu[u].w};
#pragma unroll
          for (int j = 0; j < kRowsPerPass; ++j) {
            const float pr = __builtin_amdgcn_exp2f((sc[u][j] - m[j]) * c);
            l[j] += pr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[j][2 * e] = fmaf(pr, lo_f(vw[e]), o[j][2 * e]);
              o[j][2 * e + 1] = fmaf(pr, hi_f(vw[e]), o[j][2 * e + 1]);
            }
          }
        }
      }
    }
    // merge the lane groups' states through LDS
#pragma unroll
    for (int j = 0; j < kRowsPerPass; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[sg][j][part * 8 + e] = o[j][e];
      if (part == 0) {
        red_ml[sg][j][0] = m[j];
        red_ml[sg][j][1] = l[j];
      }
    }
    __syncthreads();
    for (int x = tid; x < nr * D; x += kWaves * 64) {
      const int j = x / D, d = x % D;
      float mm = -INFINITY;
      for (int g = 0; g < NSG; ++g) mm = fmaxf(mm, red_ml[g][j][0]);
      float lt = 0.f, ot = 0.f;
      for (int g = 0; g < NSG; ++g) {
        const float mg = red_ml[g][j][0];
        if (mg == -INFINITY) continue;   // a group that saw no key
        const float w = __builtin_amdgcn_exp2f((mg - mm) * c);
        lt += red_ml[g][j][1] * w;
        ot += red_o[g][j][d] * w;
      }
      const int hh = k * G + h0 + j;
      const int64_t ro = ((int64_t)r * BW + b) * p.Hq + hh;
      if constexpr (TOKENS) {
        p.tok_o[ro * D + d] = ot;
        if (d == 0) {
          p.tok_ml[ro * 2 + 0] = mm;
          p.tok_ml[ro * 2 + 1] = lt;
        }
      } else {
        og[ro * D + d] = __builtin_bit_cast(uint16_t, (__bf16)(ot / lt));
      }
    }
    __syncthreads();
  }
}

}  // namespace

int per_beam_lds_bytes(int D) {
  return D == 64 ? (int)sizeof(PerBeamLds<64>) : (int)sizeof(PerBeamLds<128>);
}

hipError_t launch_decode_per_beam_bf16(const DecodeParams &p, hipStream_t stream,
                                       LaunchEvents ev) {
  const int64_t grid = (int64_t)p.R * p.BW * p.Hkv;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  auto go = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0u, stream,
                            ev.start, ev.stop, 0u, p);
    else
      hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  };
  if (p.D == 64)
    go(decode_per_beam_kernel<64, false>);
  else if (p.D == 128)
    go(decode_per_beam_kernel<128, false>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_token_partials_bf16(const DecodeParams &p, hipStream_t stream,
                                      LaunchEvents ev) {
  const int64_t grid = (int64_t)p.R * p.BW * p.Hkv;
  if (grid > 0x7fffffff || !p.anc || !p.tok_ml || !p.tok_o) return hipErrorInvalidConfiguration;
  auto go = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0u, stream,
                            ev.start, ev.stop, 0u, p);
    else
      hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  };
  if (p.D == 64)
    go(decode_per_beam_kernel<64, true>);
  else if (p.D == 128)
    go(decode_per_beam_kernel<128, true>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace xattn
