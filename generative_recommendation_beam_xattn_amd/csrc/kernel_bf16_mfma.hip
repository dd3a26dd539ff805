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

// Both halves of the wave hold complementary parts of a row's statistics
// (lane l and lane l ^ 32).  v_permlane32_swap exchanges the halves on the
// VALU; combining the two results symmetrically gives every lane the pair's
// max or sum.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Workgroups are dispatched to the 8 XCDs round-robin.  Giving each XCD a
// contiguous range of logical blocks keeps the row blocks of one
// (request, KV head) on one XCD, where they share its L2.
__device__ inline int xcd_logical_block(int b, int n) {
  const int xcd = b & 7, j = b >> 3;
  const int per = n >> 3, extra = n & 7;
  return xcd * per + min(xcd, extra) + j;
}

// A row's running maximum is only raised when a tile exceeds it by more
// than 2^8 in the exp2 domain; until then p = exp2(s - m) may exceed 1 (by
// at most 256), which fp32 sums and bf16 P hold without loss of range.
constexpr float kLazyRescaleLog2 = 8.0f;

// LDS layout of one workgroup: two K tiles [KT][D + KPAD] and two V^T tiles
// [D][KT + VPAD] (double buffered).  After the last tile the same bytes hold
// the partial states the key halves exchange.
template <int D>
struct TileLds {
  static constexpr int kPitch = D + KPAD;
  static constexpr int vPitch = KT + VPAD;
  static constexpr int kBytes = KT * kPitch * 2;
  static constexpr int vBytes = D * vPitch * 2;
  static constexpr int bytes = 2 * (kBytes + vBytes);
  __device__ static uint16_t *k(uint8_t *base, int buf) {
    return reinterpret_cast<uint16_t *>(base + buf * kBytes);
  }
  __device__ static uint16_t *vt(uint8_t *base, int buf) {
    return reinterpret_cast<uint16_t *>(base + 2 * kBytes + buf * vBytes);
  }
};

// Staging registers of one thread for one shared K/V tile.  K is moved in
// 16-byte chunks; V in blocks of 4 keys x 8 dims that are transposed in
// registers on the way into the V^T tile.  With 8 waves, the lower half of
// the workgroup moves K and the upper half moves V.
template <int D, int NT>
struct TileStage {
  static constexpr bool kSplitRoles = NT >= 512;
  static constexpr int kThreads = kSplitRoles ? NT / 2 : NT;
  static constexpr int KCH = KT * D / 8;
  static constexpr int VBL = KT * D / 32;
  static constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  static constexpr int VPT = (VBL + kThreads - 1) / kThreads;
  // one register file for both roles when they are split across threads
  static constexpr int NREG = kSplitRoles ? (KPT > 4 * VPT ? KPT : 4 * VPT) : KPT + 4 * VPT;
  static constexpr int VOFF = kSplitRoles ? 0 : KPT;
  uint4 reg[NREG];
  __device__ uint4 &k(int i) { return reg[i]; }
  __device__ uint4 &v(int i, int e) { return reg[VOFF + 4 * i + e]; }
  __device__ const uint4 &k(int i) const { return reg[i]; }
  __device__ const uint4 &v(int i, int e) const { return reg[VOFF + 4 * i + e]; }
};

template <int D, int NT>
__device__ __forceinline__ void tile_load(TileStage<D, NT> &st, int tid, const uint16_t *skg,
                                          const uint16_t *svg, int key0, int L) {
  using S = TileStage<D, NT>;
  // Rows past the prompt are clamped to its last row (always in bounds):
  // their scores are masked and their probabilities are exactly zero.
  const bool do_k = !S::kSplitRoles || tid < S::kThreads;
  const bool do_v = !S::kSplitRoles || tid >= S::kThreads;
  const int t = S::kSplitRoles ? tid % S::kThreads : tid;
  if (do_k) {
#pragma unroll
    for (int i = 0; i < S::KPT; ++i) {
      const int ch = t + i * S::kThreads;
      if (S::KCH % S::kThreads == 0 || ch < S::KCH) {
        const int key = min(key0 + ch / (D / 8), L - 1);
        st.k(i) = *reinterpret_cast<const uint4 *>(skg + (int64_t)key * D + (ch % (D / 8)) * 8);
      }
    }
  }
  if (do_v) {
#pragma unroll
    for (int i = 0; i < S::VPT; ++i) {
      const int bl = t + i * S::kThreads;
      if (S::VBL % S::kThreads == 0 || bl < S::VBL) {
        const int dc = bl % (D / 8);
        const int key = key0 + 4 * (bl / (D / 8));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st.v(i, e) = *reinterpret_cast<const uint4 *>(
              svg + (int64_t)min(key + e, L - 1) * D + dc * 8);
      }
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void tile_store(const TileStage<D, NT> &st, int tid, uint8_t *lds,
                                           int buf) {
  using S = TileStage<D, NT>;
  using T = TileLds<D>;
  const bool do_k = !S::kSplitRoles || tid < S::kThreads;
  const bool do_v = !S::kSplitRoles || tid >= S::kThreads;
  const int t = S::kSplitRoles ? tid % S::kThreads : tid;
  uint16_t *kl = T::k(lds, buf);
  uint16_t *vl = T::vt(lds, buf);
  if (do_k) {
#pragma unroll
    for (int i = 0; i < S::KPT; ++i) {
      const int ch = t + i * S::kThreads;
      if (S::KCH % S::kThreads == 0 || ch < S::KCH)
        *reinterpret_cast<uint4 *>(kl + (ch / (D / 8)) * T::kPitch + (ch % (D / 8)) * 8) =
            st.k(i);
    }
  }
  if (do_v) {
#pragma unroll
    for (int i = 0; i < S::VPT; ++i) {
      const int bl = t + i * S::kThreads;
      if (S::VBL % S::kThreads == 0 || bl < S::VBL) {
        const int dc = bl % (D / 8);
        const int pos = vt_pos(4 * (bl / (D / 8)));
        const uint4 r0 = st.v(i, 0), r1 = st.v(i, 1), r2 = st.v(i, 2), r3 = st.v(i, 3);
        const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
        const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
        const uint32_t w2[4] = {r2.x, r2.y, r2.z, r2.w};
        const uint32_t w3[4] = {r3.x, r3.y, r3.z, r3.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dims 2e and 2e+1 of the four keys
          const uint2 even = {(w0[e] & 0xffffu) | (w1[e] << 16), (w2[e] & 0xffffu) | (w3[e] << 16)};
          const uint2 odd = {(w0[e] >> 16) | (w1[e] & 0xffff0000u),
                             (w2[e] >> 16) | (w3[e] & 0xffff0000u)};
          *reinterpret_cast<uint2 *>(vl + (dc * 8 + 2 * e) * T::vPitch + pos) = even;
          *reinterpret_cast<uint2 *>(vl + (dc * 8 + 2 * e + 1) * T::vPitch + pos) = odd;
        }
      }
    }
  }
}

// Workgroup = RG row groups x KSPLIT key halves, one wave each.  A row group
// owns QB blocks of 32 query rows; with KSPLIT = 2 the two waves of a row
// group take the two 32-key halves of every 64-key tile and merge their
// online-softmax states through LDS at the end.
template <int D, int RG, int QB, int KSPLIT, bool TAPS>
__global__ __launch_bounds__(RG * KSPLIT * 64) void decode_bf16_kernel(DecodeParams p) {
  constexpr int WAVES = RG * KSPLIT;
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = RG * QB * 32;
  constexpr int NKS = D / 16;           // k-steps of the QK contraction
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int NKB = 2 / KSPLIT;       // 32-key blocks per wave per tile
  using T = TileLds<D>;

  __shared__ __attribute__((aligned(16))) uint8_t lds[T::bytes];
  extern __shared__ int32_t anc_lds[];  // [beams of the block][step + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = wave % RG;     // row group
  const int kh = wave / RG;     // key half
  const int hl = lane >> 5;     // lane half
  const int ql = lane & 31;     // query (B/C column) or A-operand row of this lane

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rb = lb % p.n_rb;
  const int unit = lb / p.n_rb;
  const int r = unit / p.Hkv;
  const int k = unit % p.Hkv;
  const int G = p.G, BW = p.BW, step = p.step;
  const int L = clampi(p.prompt_len[r], 0, p.Lmax);
  const float c = p.scale_log2;
  // in raw dot-product units; the debug variant reports the stages' true
  // maxima, so it raises m on every increase
  const float thr = TAPS ? 0.f : kLazyRescaleLog2 / c;

  const int row0 = rb * ROWS;
  const int b_lo = row0 / G;
  const int nb = min(BW - b_lo, (ROWS - 1) / G + 2);
  const int n_tiles = (L + KT - 1) / KT;

  // ---- loads that depend on nothing: q rows, shared tile 0
  const uint16_t *qg = static_cast<const uint16_t *>(p.q);
  uint16_t *og = static_cast<uint16_t *>(p.out);
  bf16x8 qf[QB][NKS];
  int beam[QB];
  int64_t qoff[QB];
  bool valid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = row0 + (rg * QB + qb) * 32 + ql;
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
  const uint16_t *skg = static_cast<const uint16_t *>(p.shared_k) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *svg = static_cast<const uint16_t *>(p.shared_v) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  TileStage<D, NT> stage;
  if (n_tiles > 0) tile_load<D, NT>(stage, tid, skg, svg, 0, L);

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
  if (n_tiles > 0) tile_store<D, NT>(stage, tid, lds, 0);
  __syncthreads();  // ancestor slots and tile 0 visible
  if (n_tiles > 1) tile_load<D, NT>(stage, tid, skg, svg, KT, L);

  // ---- Unshared stage: the beam's token at every level.  The debug variant
  // keeps it in key half 0; otherwise the key halves take alternate levels
  // (their partial states are merged with the rest at the end).
  float m[QB], l[QB];
  f32x16 O[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) O[qb][db] = f32x16{};
  }
  if (!TAPS || kh == 0) {
    const int t_first = TAPS ? 0 : kh;
    const int t_stride = TAPS ? 1 : KSPLIT;
    const uint16_t *ukg = static_cast<const uint16_t *>(p.unshared_k) +
                          ((int64_t)r * p.Hkv + k) * p.S * BW * D;
    const uint16_t *uvg = static_cast<const uint16_t *>(p.unshared_v) +
                          ((int64_t)r * p.Hkv + k) * p.S * BW * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int bi = beam[qb] - b_lo;
      for (int t = t_first; t <= step; t += t_stride) {
        const int slot = p.anc ? clampi(p.anc[((int64_t)r * (step + 1) + t) * BW + beam[qb]], 0,
                                        BW - 1)
                               : anc_lds[bi * (step + 1) + t];
        const int64_t roff = ((int64_t)t * BW + slot) * D;
        uint4 kr[NKS];
        uint2 vr[NDB][4];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          kr[ks] = *reinterpret_cast<const uint4 *>(ukg + roff + ks * 16 + hl * 8);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            vr[db][j] = *reinterpret_cast<const uint2 *>(uvg + roff + db * 32 + 8 * j + 4 * hl);
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          part = dot8(__builtin_bit_cast(uint4, qf[qb][ks]), kr[ks], part);
        const float sc = pair_sum(part);
        const float mn = fmaxf(m[qb], sc);
        const float alpha = __builtin_amdgcn_exp2f((m[qb] - mn) * c);  // 0 while m is -inf
        const float pr = __builtin_amdgcn_exp2f((sc - mn) * c);
        l[qb] = l[qb] * alpha + pr;
        m[qb] = mn;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint2 v = vr[db][j];
            O[qb][db][4 * j + 0] = fmaf(O[qb][db][4 * j + 0], alpha, pr * lo_bf16(v.x));
            O[qb][db][4 * j + 1] = fmaf(O[qb][db][4 * j + 1], alpha, pr * hi_bf16(v.x));
            O[qb][db][4 * j + 2] = fmaf(O[qb][db][4 * j + 2], alpha, pr * lo_bf16(v.y));
            O[qb][db][4 * j + 3] = fmaf(O[qb][db][4 * j + 3], alpha, pr * hi_bf16(v.y));
          }
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
      if (kh == 0) {
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

  // ---- Shared stage: tile `it` is in LDS buffer it & 1 and tile it + 1 is
  // in flight in registers while tile it is consumed
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int key0 = it * KT;
    const uint16_t *kl = T::k(lds, buf);
    const uint16_t *vl = T::vt(lds, buf);

    // S^T = K . Q^T for this wave's 32-key block(s) of the tile
    f32x16 sacc[NKB][QB];
#pragma unroll
    for (int i = 0; i < NKB; ++i)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[i][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int i = 0; i < NKB; ++i) {
        const int kb = kh * NKB + i;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kl + (kb * 32 + ql) * T::kPitch +
                                                           ks * 16 + hl * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[i][qb] = mfma(a, qf[qb][ks], sacc[i][qb]);
      }
    }

    // online softmax (scores stay in raw dot units; exp2 with scale*log2e)
    const bool tail = key0 + KT > L;
    bf16x8 pf[QB][2 * NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < NKB; ++i) {
        const int kb = kh * NKB + i;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (tail) {
            const int key = key0 + kb * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
            if (key >= L) sacc[i][qb][e] = -INFINITY;
          }
          tmax = fmaxf(tmax, sacc[i][qb][e]);
        }
      }
      tmax = pair_max(tmax);
      if (__any(tmax > m[qb] + thr)) {
        const float mn = fmaxf(m[qb], tmax);
        const float alpha = __builtin_amdgcn_exp2f((m[qb] - mn) * c);
        m[qb] = mn;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) O[qb][db] *= alpha;
      }
      // a key half can see only masked keys: m stays -inf and p = 0
      const float mc = m[qb] == -INFINITY ? 0.f : m[qb] * c;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < NKB; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[i][qb][e], c, -mc));
          sacc[i][qb][e] = pe;
          lsum += pe;
        }
      }
      l[qb] += lsum;
#pragma unroll
      for (int j = 0; j < 2 * NKB; ++j) pf[qb][j] = to_bf16x8(sacc[j >> 1][qb], 8 * (j & 1));
    }

    // O^T += V^T . P^T over this wave's keys
#pragma unroll
    for (int j = 0; j < 2 * NKB; ++j) {
      const int ps = 2 * kh * NKB + j;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vl + (db * 32 + ql) * T::vPitch +
                                                           ps * 16 + hl * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) O[qb][db] = mfma(a, pf[qb][j], O[qb][db]);
      }
    }

    if (it + 1 < n_tiles) tile_store<D, NT>(stage, tid, lds, buf ^ 1);
    __syncthreads();
    if (it + 2 < n_tiles) tile_load<D, NT>(stage, tid, skg, svg, key0 + 2 * KT, L);
  }

  // ---- the second key half hands its state to the first through LDS
  if constexpr (KSPLIT == 2) {
    float *xo = reinterpret_cast<float *>(lds) + rg * (QB * (NDB * 16 + 2) * 64);
    if (kh == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float *dst = xo + qb * (NDB * 16 + 2) * 64;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) dst[(db * 16 + e) * 64 + lane] = O[qb][db][e];
        dst[(NDB * 16) * 64 + lane] = m[qb];
        dst[(NDB * 16 + 1) * 64 + lane] = l[qb];
      }
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float *src = xo + qb * (NDB * 16 + 2) * 64;
      const float m2 = src[(NDB * 16) * 64 + lane];
      const float l2 = src[(NDB * 16 + 1) * 64 + lane];
      float a1 = 1.f, a2 = 0.f;
      if (m2 > m[qb]) {
        a1 = __builtin_amdgcn_exp2f((m[qb] - m2) * c);  // 0 when m is -inf
        a2 = 1.f;
        m[qb] = m2;
      } else if (m2 != -INFINITY) {
        a2 = __builtin_amdgcn_exp2f((m2 - m[qb]) * c);
      }
      l[qb] = l[qb] * a1 + l2 * a2;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          O[qb][db][e] = O[qb][db][e] * a1 + src[(db * 16 + e) * 64 + lane] * a2;
    }
  }

  // ---- Merge / epilogue
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(l[qb]);
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

template <int D, int RG, int QB, int KSPLIT, bool TAPS>
hipError_t launch_cfg(const DecodeParams &p0, hipStream_t stream) {
  constexpr int ROWS = RG * QB * 32;
  DecodeParams p = p0;
  p.n_rb = (p.M + ROWS - 1) / ROWS;
  const int64_t grid = (int64_t)p.R * p.Hkv * p.n_rb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  size_t dyn = 0;
  if (p.anc == nullptr) {
    const int nb = min(p.BW, (ROWS - 1) / p.G + 2);
    dyn = (size_t)nb * (p.step + 1) * sizeof(int32_t);
  }
  hipLaunchKernelGGL((decode_bf16_kernel<D, RG, QB, KSPLIT, TAPS>), dim3((unsigned)grid),
                     dim3(RG * KSPLIT * 64), dyn, stream, p);
  return hipGetLastError();
}

// Rows per workgroup: 32 (1 wave) or 64 (2 waves) for few query rows per
// (request, KV head); otherwise 128 rows in 4 row groups x 2 key halves.
int rows_per_block(int M) { return M <= 32 ? 32 : (M <= 64 ? 64 : 128); }

template <int D>
hipError_t launch_d(const DecodeParams &p, bool taps, hipStream_t stream) {
  const int rows = rows_per_block(p.M);
  if (taps) {
    if (rows == 32) return launch_cfg<D, 1, 1, 1, true>(p, stream);
    if (rows == 64) return launch_cfg<D, 2, 1, 1, true>(p, stream);
    return launch_cfg<D, 4, 1, 2, true>(p, stream);
  }
  if (rows == 32) return launch_cfg<D, 1, 1, 1, false>(p, stream);
  if (rows == 64) return launch_cfg<D, 2, 1, 1, false>(p, stream);
  return launch_cfg<D, 4, 1, 2, false>(p, stream);
}

}  // namespace

int bf16_rows_per_block(const DecodeParams &p) { return rows_per_block(p.M); }

hipError_t launch_decode_bf16(const DecodeParams &p, bool taps, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, taps, stream);
  if (p.D == 128) return launch_d<128>(p, taps, stream);
  return hipErrorInvalidValue;
}

}  // namespace xattn
