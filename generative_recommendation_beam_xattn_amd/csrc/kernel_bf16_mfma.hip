// Staged decode attention, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Implements the xAttention operator of the xGR technical summary
// (gist.science, paper 2512.11529), section 2.1: a Shared stage over the
// request's prompt KV (stored once per request and read once for all of
// its beams), an Unshared stage over each beam's own generated tokens
// (one row per level and slot, reached through the parent indices, never
// copied), and an OnlineSoftmax merge of the two.
//
// Work decomposition.  One workgroup owns a block of ROWS query rows of one
// (request r, KV head k).  The M = BW * G rows of (r, k) are ordered
// (beam, head-in-group), so every row of the block reads the same shared
// K/V stream: each K/V tile is staged once in LDS and contracted against all
// rows of the block on the matrix cores.  Each wave owns QB blocks of 32
// rows.
//
// Shared stage, per 64-key tile:
//   S^T (keys x queries) = K (keys x D) . Q^T (D x queries)
//   online softmax on S^T (a lane holds one query, 16 keys per 32-key block,
//   so row statistics need one cross-lane exchange)
//   O^T (D x queries) += V^T (D x keys) . P^T (keys x queries)
// all with v_mfma_f32_32x32x16_bf16.  The P^T operand is taken straight from
// the S^T accumulators; the key order inside a 64-key tile is permuted so
// that the V^T tile in LDS lines up with it (see vt_pos()).
//
// Unshared stage: each row's s+1 ancestor tokens are gathered from global
// memory by the lanes that hold that row (VALU dot products in fp32).  Its
// (max, sum, output) seed the online-softmax state before the shared tiles
// stream in, so the Merge is the first online-softmax update.  The debug
// variant (TAPS) instead keeps the two stages apart, writes each stage's
// (m, l, o) and merges them explicitly at the end.
#include "xattn_internal.h"

namespace xattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;    // keys per shared-stage tile
constexpr int KPAD = 8;   // bf16 elements of padding per K row in LDS
constexpr int VPAD = 8;   // bf16 elements of padding per V^T row in LDS

__device__ inline float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ inline float dot8(uint4 a, uint4 b, float acc) {
  acc = fmaf(lo_bf16(a.x), lo_bf16(b.x), acc);
  acc = fmaf(hi_bf16(a.x), hi_bf16(b.x), acc);
  acc = fmaf(lo_bf16(a.y), lo_bf16(b.y), acc);
  acc = fmaf(hi_bf16(a.y), hi_bf16(b.y), acc);
  acc = fmaf(lo_bf16(a.z), lo_bf16(b.z), acc);
  acc = fmaf(hi_bf16(a.z), hi_bf16(b.z), acc);
  acc = fmaf(lo_bf16(a.w), lo_bf16(b.w), acc);
  acc = fmaf(hi_bf16(a.w), hi_bf16(b.w), acc);
  return acc;
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 to_bf16x8(const f32x16 &v, int off) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[off + e];
  return r;
}

// Position of key `key` (0..63) of a tile inside a V^T row in LDS.
// In the S^T accumulator of a 32-key block, the lane in half h holds keys
// 8j + 4h + i (j, i = 0..3).  The PV contraction over k-step ps (16 keys)
// feeds the lane's accumulator entries 8*(ps%2) .. +7 of block ps/2, i.e.
// keys 32*(ps/2) + 16*(ps%2) + 8*(e/4) + 4h + e%4 for e = 0..7.  Storing key
// bits [5 4 3 2 1:0] at position bits [5 4 2 3 1:0] (bits 2 and 3 swapped)
// puts exactly those eight keys at positions 16*ps + 8h + e.
__device__ inline int vt_pos(int key) {
  return (key & ~0xC) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ inline int clampi(int v, int lo, int hi) { return min(max(v, lo), hi); }

template <int D, int WAVES, int QB, bool TAPS>
__global__ __launch_bounds__(WAVES * 64) void decode_bf16_kernel(DecodeParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = WAVES * QB * 32;
  constexpr int NKS = D / 16;           // k-steps of the QK contraction
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int KCH = KT * D / 8;       // 16-byte K chunks per tile
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VBL = KT * D / 32;      // (4 keys x 8 dims) V blocks per tile
  constexpr int VPT = (VBL + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT][D + KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D][KT + VPAD];
  extern __shared__ int32_t anc_lds[];  // [beams of the block][step + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;   // lane half
  const int ql = lane & 31;   // query (B/C column) or A-operand row of this lane

  const int rb = blockIdx.x % p.n_rb;
  const int unit = blockIdx.x / p.n_rb;
  const int r = unit / p.Hkv;
  const int k = unit % p.Hkv;
  const int G = p.G, BW = p.BW, step = p.step;
  const int L = clampi(p.prompt_len[r], 0, p.Lmax);
  const float c = p.scale_log2;

  const int row0 = rb * ROWS;
  const int b_lo = row0 / G;
  const int nb = min(BW - b_lo, (ROWS - 1) / G + 2);

  // ---- ancestor slots of the block's beams (short chains: walked here)
  if (p.anc == nullptr) {
    const int32_t *par = p.parent_idx + (int64_t)r * p.S * BW;
    for (int i = tid; i < nb; i += NT) {
      int a = b_lo + i;
      int32_t *dst = anc_lds + i * (step + 1);
      dst[step] = a;
      for (int t = step; t >= 1; --t) {
        a = clampi(par[(int64_t)t * BW + a], 0, BW - 1);
        dst[t - 1] = a;
      }
    }
  }

  // ---- this lane's query rows
  const uint16_t *qg = static_cast<const uint16_t *>(p.q);
  uint16_t *og = static_cast<uint16_t *>(p.out);
  bf16x8 qf[QB][NKS];
  int beam[QB];
  int64_t qoff[QB];
  bool valid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = row0 + (wave * QB + qb) * 32 + ql;
    valid[qb] = row < p.M;
    const int rr = valid[qb] ? row : p.M - 1;
    beam[qb] = rr / G;
    const int h = k * G + rr % G;
    qoff[qb] = (((int64_t)r * BW + beam[qb]) * p.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[qb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                  qg + qoff[qb] + ks * 16 + hl * 8));
  }
  __syncthreads();  // ancestor slots visible

  // ---- Unshared stage: the beam's token at every level 0..step
  const uint16_t *ukg = static_cast<const uint16_t *>(p.unshared_k) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  const uint16_t *uvg = static_cast<const uint16_t *>(p.unshared_v) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  float m[QB], l[QB];
  f32x16 O[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) O[qb][db] = f32x16{};
    const int bi = beam[qb] - b_lo;
    for (int t = 0; t <= step; ++t) {
      const int slot = p.anc ? clampi(p.anc[((int64_t)r * (step + 1) + t) * BW + beam[qb]], 0,
                                      BW - 1)
                             : anc_lds[bi * (step + 1) + t];
      const int64_t roff = ((int64_t)t * BW + slot) * D;
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        part = dot8(__builtin_bit_cast(uint4, qf[qb][ks]),
                    *reinterpret_cast<const uint4 *>(ukg + roff + ks * 16 + hl * 8), part);
      const float sc = part + __shfl_xor(part, 32);
      const float mn = fmaxf(m[qb], sc);
      const float alpha = __builtin_amdgcn_exp2f((m[qb] - mn) * c);
      const float pr = __builtin_amdgcn_exp2f((sc - mn) * c);
      l[qb] = l[qb] * alpha + pr;
      m[qb] = mn;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 v = *reinterpret_cast<const uint2 *>(uvg + roff + db * 32 + 8 * j + 4 * hl);
          O[qb][db][4 * j + 0] = fmaf(O[qb][db][4 * j + 0], alpha, pr * lo_bf16(v.x));
          O[qb][db][4 * j + 1] = fmaf(O[qb][db][4 * j + 1], alpha, pr * hi_bf16(v.x));
          O[qb][db][4 * j + 2] = fmaf(O[qb][db][4 * j + 2], alpha, pr * lo_bf16(v.y));
          O[qb][db][4 * j + 3] = fmaf(O[qb][db][4 * j + 3], alpha, pr * hi_bf16(v.y));
        }
      }
    }
  }

  const int64_t n_rows_all = (int64_t)p.R * BW * p.Hq;
  // Debug variant: the Unshared partial is kept on its own (mu, lu, Ou),
  // written as stage 1, and the running state restarts for the Shared stage.
  float mu[QB], lu[QB];
  f32x16 Ou[TAPS ? QB : 1][TAPS ? NDB : 1];
  if constexpr (TAPS) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mu[qb] = m[qb];
      lu[qb] = l[qb];
      const float inv = 1.f / l[qb];
#pragma unroll
      for (int db = 0; db < NDB; ++db) Ou[qb][db] = O[qb][db] * inv;
      const int64_t ri = qoff[qb] / D;
      if (valid[qb]) {
        if (p.stage_ml && hl == 0) {
          p.stage_ml[(n_rows_all + ri) * 2 + 0] = m[qb] * p.scale;
          p.stage_ml[(n_rows_all + ri) * 2 + 1] = l[qb];
        }
        if (p.stage_o) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              p.stage_o[(n_rows_all + ri) * D + db * 32 + 8 * (e / 4) + 4 * hl + e % 4] =
                  Ou[qb][db][e];
        }
      }
      m[qb] = -INFINITY;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[qb][db] = f32x16{};
    }
  } else {
    // Seeded state: both lanes of a pair hold the full unshared sum; keep it
    // in one lane so the final pair-sum counts it once.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l[qb] = hl == 0 ? l[qb] : 0.f;
  }

  // ---- Shared stage
  const uint16_t *skg = static_cast<const uint16_t *>(p.shared_k) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *svg = static_cast<const uint16_t *>(p.shared_v) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const int n_tiles = (L + KT - 1) / KT;
  uint4 kreg[KPT];
  uint4 vreg[VPT][4];

  auto load_tile = [&](int key0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ch = tid + i * NT;
      if (ch < KCH) {
        const int key = key0 + ch / (D / 8);
        kreg[i] = key < L ? *reinterpret_cast<const uint4 *>(skg + (int64_t)key * D +
                                                              (ch % (D / 8)) * 8)
                          : uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int bl = tid + i * NT;
      if (bl < VBL) {
        const int dc = bl % (D / 8);
        const int key = key0 + 4 * (bl / (D / 8));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vreg[i][e] = key + e < L ? *reinterpret_cast<const uint4 *>(
                                         svg + (int64_t)(key + e) * D + dc * 8)
                                   : uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ch = tid + i * NT;
      if (ch < KCH)
        *reinterpret_cast<uint4 *>(&k_lds[buf][ch / (D / 8)][(ch % (D / 8)) * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int bl = tid + i * NT;
      if (bl < VBL) {
        const int dc = bl % (D / 8);
        const int pos = vt_pos(4 * (bl / (D / 8)));
        const uint32_t w0[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
        const uint32_t w1[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
        const uint32_t w2[4] = {vreg[i][2].x, vreg[i][2].y, vreg[i][2].z, vreg[i][2].w};
        const uint32_t w3[4] = {vreg[i][3].x, vreg[i][3].y, vreg[i][3].z, vreg[i][3].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dims 2e and 2e+1 of the four keys
          const uint2 even = {(w0[e] & 0xffffu) | (w1[e] << 16), (w2[e] & 0xffffu) | (w3[e] << 16)};
          const uint2 odd = {(w0[e] >> 16) | (w1[e] & 0xffff0000u),
                             (w2[e] >> 16) | (w3[e] & 0xffff0000u)};
          *reinterpret_cast<uint2 *>(&vt_lds[buf][dc * 8 + 2 * e][pos]) = even;
          *reinterpret_cast<uint2 *>(&vt_lds[buf][dc * 8 + 2 * e + 1][pos]) = odd;
        }
      }
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int key0 = it * KT;
    if (it + 1 < n_tiles) load_tile(key0 + KT);

    // S^T = K . Q^T for the two 32-key blocks of the tile
    f32x16 sacc[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&k_lds[buf][kb * 32 + ql][ks * 16 + hl * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mfma(a, qf[qb][ks], sacc[kb][qb]);
      }
    }

    // online softmax (scores stay in raw dot units; exp2 with scale*log2e)
    const bool tail = key0 + KT > L;
    bf16x8 pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (tail) {
            const int key = key0 + kb * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
            if (key >= L) sacc[kb][qb][e] = -INFINITY;
          }
          tmax = fmaxf(tmax, sacc[kb][qb][e]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m[qb], tmax);
      const float alpha = __builtin_amdgcn_exp2f((m[qb] - mn) * c);
      const float mc = mn * c;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][e], c, -mc));
          sacc[kb][qb][e] = pe;
          lsum += pe;
        }
      }
      l[qb] = fmaf(l[qb], alpha, lsum);
      m[qb] = mn;
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[qb][db] *= alpha;
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) pf[qb][ps] = to_bf16x8(sacc[ps >> 1][qb], 8 * (ps & 1));
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&vt_lds[buf][db * 32 + ql][ps * 16 + hl * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) O[qb][db] = mfma(a, pf[qb][ps], O[qb][db]);
      }
    }

    if (it + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- Merge / epilogue
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    if constexpr (TAPS) {
      // Shared partial (m, lt, O / lt) on its own, then the explicit
      // OnlineSoftmax merge with the Unshared partial (mu, lu, Ou).
      const int64_t ri = qoff[qb] / D;
      const float ms = m[qb];
      const float inv_s = lt > 0.f ? 1.f / lt : 0.f;
      const float mm = fmaxf(ms, mu[qb]);
      const float ws = lt > 0.f ? lt * __builtin_amdgcn_exp2f((ms - mm) * c) : 0.f;
      const float wu = lu[qb] * __builtin_amdgcn_exp2f((mu[qb] - mm) * c);
      const float inv_z = 1.f / (ws + wu);
      if (valid[qb]) {
        if (p.stage_ml && hl == 0) {
          p.stage_ml[ri * 2 + 0] = lt > 0.f ? ms * p.scale : -INFINITY;
          p.stage_ml[ri * 2 + 1] = lt;
        }
        if (p.stage_o) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              p.stage_o[ri * D + db * 32 + 8 * (e / 4) + 4 * hl + e % 4] = O[qb][db][e] * inv_s;
        }
        if (p.lse && hl == 0) p.lse[ri] = mm * p.scale + __logf(ws + wu);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        O[qb][db] = (O[qb][db] * (inv_s * ws) + Ou[qb][db] * wu) * inv_z;
    } else {
      const float inv = 1.f / lt;
      if (valid[qb] && p.lse && hl == 0) p.lse[qoff[qb] / D] = m[qb] * p.scale + __logf(lt);
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[qb][db] *= inv;
    }
    if (!valid[qb]) continue;
    uint16_t *op = og + qoff[qb];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 pk = {(__bf16)O[qb][db][4 * j + 0], (__bf16)O[qb][db][4 * j + 1],
                           (__bf16)O[qb][db][4 * j + 2], (__bf16)O[qb][db][4 * j + 3]};
        *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * j + 4 * hl) = pk;
      }
    }
  }
}

template <int D, int WAVES, int QB, bool TAPS>
hipError_t launch_cfg(const DecodeParams &p0, hipStream_t stream) {
  constexpr int ROWS = WAVES * QB * 32;
  DecodeParams p = p0;
  p.n_rb = (p.M + ROWS - 1) / ROWS;
  const int64_t grid = (int64_t)p.R * p.Hkv * p.n_rb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  size_t dyn = 0;
  if (p.anc == nullptr) {
    const int nb = min(p.BW, (ROWS - 1) / p.G + 2);
    dyn = (size_t)nb * (p.step + 1) * sizeof(int32_t);
  }
  hipLaunchKernelGGL((decode_bf16_kernel<D, WAVES, QB, TAPS>), dim3((unsigned)grid),
                     dim3(WAVES * 64), dyn, stream, p);
  return hipGetLastError();
}

struct TileChoice {
  int waves, qb;
};

TileChoice choose_tile(const DecodeParams &p) {
  if (p.M <= 32) return {1, 1};
  if (p.M <= 64) return {2, 1};
  if (p.M <= 128) return {4, 1};
  // Two 32-row blocks per wave halve the LDS traffic per MFMA; use them
  // when there are still enough workgroups to cover the 256 CUs twice.
  const int64_t blocks_qb2 = (int64_t)p.R * p.Hkv * ((p.M + 255) / 256);
  return blocks_qb2 >= 512 ? TileChoice{4, 2} : TileChoice{4, 1};
}

template <int D>
hipError_t launch_d(const DecodeParams &p, bool taps, hipStream_t stream) {
  const TileChoice t = choose_tile(p);
  if (taps) {
    // the debug variant keeps a second stage state in registers: one
    // 32-row block per wave
    if (t.waves == 1) return launch_cfg<D, 1, 1, true>(p, stream);
    if (t.waves == 2) return launch_cfg<D, 2, 1, true>(p, stream);
    return launch_cfg<D, 4, 1, true>(p, stream);
  }
  if (t.waves == 1) return launch_cfg<D, 1, 1, false>(p, stream);
  if (t.waves == 2) return launch_cfg<D, 2, 1, false>(p, stream);
  if (t.qb == 1) return launch_cfg<D, 4, 1, false>(p, stream);
  return launch_cfg<D, 4, 2, false>(p, stream);
}

}  // namespace

int bf16_rows_per_block(const DecodeParams &p) {
  const TileChoice t = choose_tile(p);  // xattn_decode's tiling
  return t.waves * t.qb * 32;
}

hipError_t launch_decode_bf16(const DecodeParams &p, bool taps, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, taps, stream);
  if (p.D == 128) return launch_d<128>(p, taps, stream);
  return hipErrorInvalidValue;
}

}  // namespace xattn
