// Staged decode attention, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Implements the xAttention operator of the xGR technical summary
// (gist.science, paper 2512.11529), section 2.1: a Shared stage over the
// request's prompt KV (stored once per request and read once for all of
// its beams), an Unshared stage over each beam's own generated tokens
// (one row per level and slot, reached through the parent indices, never
// copied), and an OnlineSoftmax merge of the two.
//
// Work decomposition.  One workgroup owns a block of 32 * RG query rows of
// one (request r, KV head k).  The M = BW * G rows of (r, k) are ordered
// (beam, head-in-group), so every row of the block reads the same shared
// K/V stream: each K/V tile is brought into LDS once and contracted against
// all rows of the block on the matrix cores.  The workgroup has RG row
// groups x KSPLIT key halves, one wave each; with KSPLIT = 2 the two waves
// of a row group take the two 32-key halves of every 64-key tile and merge
// their online-softmax states through LDS at the end (two waves per SIMD,
// so one wave's softmax overlaps the other's MFMAs).
//
// Shared stage, per 64-key tile:
//   S^T (keys x queries) = K (keys x D) . Q^T (D x queries)
//   online softmax on S^T (a lane holds one query and 16 keys per 32-key
//   block; row statistics need one exchange between the wave's halves)
//   O^T (D x queries) += V^T (D x keys) . P^T (keys x queries)
// all with v_mfma_f32_32x32x16_bf16.  The P^T operand is taken straight
// from the S^T accumulators.
//
// Tile pipeline.  Tiles are copied HBM -> LDS by global_load_lds (16 bytes
// per lane, no registers involved) into a ring of NSTAGE buffers, NSTAGE-1
// tiles ahead of the one being consumed.  K and V tiles are stored
// row-major with the 16-byte slots of each row permuted by an XOR swizzle
// (TileGeom::swz) so that the K fragment reads (ds_read_b128) and the V^T
// fragment reads (ds_read_b64_tr_b16, which transposes 4x4 blocks of bf16
// across lanes) are free of bank conflicts.
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
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int KT = 64;      // keys per shared-stage tile
constexpr int NSTAGE = 4;   // LDS ring depth (tiles in flight = NSTAGE - 1)

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

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8) waiting for vmcnt <= VM and lgkmcnt == 0.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier that also orders this wave's LDS accesses in the
// compiler, without the vmcnt(0) a full fence would impose on the tile
// copies still in flight.  Callers wait for the copies they need first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Geometry of one LDS stage: a K tile then a V tile, each KT rows of D
// bf16, row-major, with the 16-byte slots of row r permuted by swz(r).
template <int D>
struct TileGeom {
  static constexpr int RB = D * 2;                 // bytes per row
  static constexpr int SLOTS = D / 8;              // 16-byte slots per row
  static constexpr int TILE_BYTES = KT * RB;       // one K (or V) tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int ROWS_PER_COPY = 1024 / RB;  // rows one wave-wide 16-byte copy fills
  static constexpr int COPIES = 2 * TILE_BYTES / 1024;  // wave-wide copies per stage (K and V)
  // Slot permutation.  D = 128 (16 slots): swap the two 2-bit fields of
  // r mod 16.  D = 64 (8 slots, 2 rows per 256 bytes): from u = r >> 1,
  // slot bit 2 = u bit 0, slot bits 1:0 = u bits 2:1.  Either way the 16
  // rows a ds_read_b128 touches map to distinct banks, and so do the 4 rows
  // x 4 slots a transposing 64-bit read touches.
  __device__ static int swz(int r) {
    if constexpr (D == 128) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
      const int u = r >> 1;
      return ((u & 1) << 2) | ((u >> 1) & 3);
    }
  }
};

// Copy the K and V tile starting at key0 into `stage` (this wave's share of
// the COPIES wave-wide copies).  Rows past the prompt are clamped to its
// last row (always in bounds): their scores are masked and their
// probabilities are exactly zero.
template <int D, int WAVES>
__device__ __forceinline__ void tile_copy(uint8_t *stage, const uint16_t *skg, const uint16_t *svg,
                                          int key0, int L, int wave, int lane) {
  using Gm = TileGeom<D>;
  constexpr int NQ = Gm::TILE_BYTES / 1024;   // copies per K (or V) tile
  constexpr int PER = Gm::COPIES / WAVES;
  static_assert(Gm::COPIES % WAVES == 0, "copies must split evenly over the waves");
  const int sub = lane / Gm::SLOTS;
  const int slot = lane % Gm::SLOTS;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int qi = wave * PER + i;
    const bool is_v = qi >= NQ;
    const int q = is_v ? qi - NQ : qi;
    const int row = q * Gm::ROWS_PER_COPY + sub;
    const int key = min(key0 + row, L - 1);
    const uint16_t *src = (is_v ? svg : skg) + (int64_t)key * D + (slot ^ Gm::swz(row)) * 8;
    uint8_t *dst = stage + (is_v ? Gm::TILE_BYTES : 0) + q * 1024;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
  }
}

// Per-lane state of one wave's 32 query rows.
template <int D>
struct Rows {
  float m, l;
  f32x16 O[D / 32];
};

// One 64-key tile from `stage`: this wave's 32-key block(s) of S^T, the
// online-softmax update and the PV contraction.
template <int D, int KSPLIT>
__device__ __forceinline__ void consume_tile(const uint8_t *stage, const bf16x8 (&qf)[D / 16],
                                             Rows<D> &st, int kh, int key0, int L, float c,
                                             float thr, int lane) {
  using Gm = TileGeom<D>;
  constexpr int NKS = D / 16, NDB = D / 32, NKB = 2 / KSPLIT;
  const int hl = lane >> 5, ql = lane & 31;

  // S^T = K . Q^T
  const int kswz = Gm::swz(ql);  // rows kb * 32 + ql share the permutation of row ql
  f32x16 sacc[NKB];
#pragma unroll
  for (int i = 0; i < NKB; ++i) sacc[i] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int i = 0; i < NKB; ++i) {
      const int kb = kh * NKB + i;
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
          stage + (kb * 32 + ql) * Gm::RB + (((2 * ks + hl) ^ kswz) << 4));
      sacc[i] = mfma(a, qf[ks], sacc[i]);
    }
  }

  // online softmax (scores stay in raw dot units; exp2 with scale*log2e)
  float tmax = -INFINITY;
  const bool tail = key0 + KT > L;
#pragma unroll
  for (int i = 0; i < NKB; ++i) {
    const int kb = kh * NKB + i;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (tail) {
        const int key = key0 + kb * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
        if (key >= L) sacc[i][e] = -INFINITY;
      }
      tmax = fmaxf(tmax, sacc[i][e]);
    }
  }
  tmax = pair_max(tmax);
  if (__any(tmax > st.m + thr)) {
    const float mn = fmaxf(st.m, tmax);
    const float alpha = __builtin_amdgcn_exp2f((st.m - mn) * c);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.O[db] *= alpha;
  }
  // a key half can see only masked keys: m stays -inf and p = 0
  const float mc = st.m == -INFINITY ? 0.f : st.m * c;
  float lsum = 0.f;
  bf16x8 pf[2 * NKB];
#pragma unroll
  for (int i = 0; i < NKB; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[i][e], c, -mc));
      sacc[i][e] = pe;
      lsum += pe;
    }
    pf[2 * i] = to_bf16x8(sacc[i], 0);
    pf[2 * i + 1] = to_bf16x8(sacc[i], 8);
  }
  st.l += lsum;

  // O^T += V^T . P^T.  For k-step ps (16 keys) the B operand of lane half
  // h holds the keys 32*(ps/2) + 16*(ps%2) + 8*e2 + 4h + (0..3), e2 = 0, 1;
  // each half-fragment of V^T is one transposing read: lane j of a 16-lane
  // group points at 4 dims of key row base + j/4, and receives 4 keys of
  // dim d0 + (lane % 16).
  const uint8_t *vt = stage + Gm::TILE_BYTES;
  const int vh = lane >> 5, vg = (lane >> 4) & 1, vj = lane & 15;
#pragma unroll
  for (int j2 = 0; j2 < 2 * NKB; ++j2) {
    const int ps = 2 * kh * NKB + j2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 half_frag[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int row = (ps >> 1) * 32 + (ps & 1) * 16 + e2 * 8 + vh * 4 + (vj >> 2);
        const int chunk = 4 * db + 2 * vg + ((vj >> 1) & 1);
        const uint8_t *addr = vt + row * Gm::RB + ((chunk ^ Gm::swz(row)) << 4) + ((vj & 1) << 3);
        half_frag[e2] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)addr);
      }
      const bf16x8 a = {half_frag[0][0], half_frag[0][1], half_frag[0][2], half_frag[0][3],
                        half_frag[1][0], half_frag[1][1], half_frag[1][2], half_frag[1][3]};
      st.O[db] = mfma(a, pf[j2], st.O[db]);
    }
  }
}

template <int D, int RG, int KSPLIT, bool TAPS>
__global__ __launch_bounds__(RG * KSPLIT * 64) void decode_bf16_kernel(DecodeParams p) {
  constexpr int WAVES = RG * KSPLIT;
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = RG * 32;
  constexpr int NKS = D / 16;           // k-steps of the QK contraction
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  using Gm = TileGeom<D>;
  constexpr int COPIES_PER_WAVE = Gm::COPIES / WAVES;

  // one LDS object per ring stage, so the compiler tracks the copies into
  // each stage separately
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[Gm::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[Gm::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[Gm::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[Gm::STAGE_BYTES];
  extern __shared__ int32_t anc_lds[];  // [beams of the block][step + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = wave % RG;     // row group
  const int kh = wave / RG;     // key half
  const int hl = lane >> 5;     // lane half
  const int ql = lane & 31;     // query (B/C column) of this lane

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

  // ---- start the tile pipeline: tiles 0 .. NSTAGE-2 in flight
  const uint16_t *skg = static_cast<const uint16_t *>(p.shared_k) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *svg = static_cast<const uint16_t *>(p.shared_v) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  if (n_tiles > 0) tile_copy<D, WAVES>(stage0, skg, svg, 0, L, wave, lane);
  if (n_tiles > 1) tile_copy<D, WAVES>(stage1, skg, svg, KT, L, wave, lane);
  if (n_tiles > 2) tile_copy<D, WAVES>(stage2, skg, svg, 2 * KT, L, wave, lane);

  // ---- this wave's query rows
  const uint16_t *qg = static_cast<const uint16_t *>(p.q);
  uint16_t *og = static_cast<uint16_t *>(p.out);
  const int row = row0 + rg * 32 + ql;
  const bool valid = row < p.M;
  const int rr = valid ? row : p.M - 1;
  const int beam = rr / G;
  const int64_t qoff = (((int64_t)r * BW + beam) * p.Hq + k * G + rr % G) * D;
  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const uint4 *>(qg + qoff + ks * 16 + hl * 8));

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
  __syncthreads();  // ancestor slots visible

  // ---- Unshared stage: the beam's token at every level.  The debug variant
  // keeps it in key half 0; otherwise the key halves take alternate levels
  // (their partial states are merged with the rest at the end).
  Rows<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) st.O[db] = f32x16{};
  if (!TAPS || kh == 0) {
    const int t_first = TAPS ? 0 : kh;
    const int t_stride = TAPS ? 1 : KSPLIT;
    const uint16_t *ukg = static_cast<const uint16_t *>(p.unshared_k) +
                          ((int64_t)r * p.Hkv + k) * p.S * BW * D;
    const uint16_t *uvg = static_cast<const uint16_t *>(p.unshared_v) +
                          ((int64_t)r * p.Hkv + k) * p.S * BW * D;
    const int bi = beam - b_lo;
    for (int t = t_first; t <= step; t += t_stride) {
      const int slot = p.anc ? clampi(p.anc[((int64_t)r * (step + 1) + t) * BW + beam], 0, BW - 1)
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
        part = dot8(__builtin_bit_cast(uint4, qf[ks]), kr[ks], part);
      const float sc = pair_sum(part);
      const float mn = fmaxf(st.m, sc);
      const float alpha = __builtin_amdgcn_exp2f((st.m - mn) * c);  // 0 while m is -inf
      const float pr = __builtin_amdgcn_exp2f((sc - mn) * c);
      st.l = st.l * alpha + pr;
      st.m = mn;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 v = vr[db][j];
          st.O[db][4 * j + 0] = fmaf(st.O[db][4 * j + 0], alpha, pr * lo_bf16(v.x));
          st.O[db][4 * j + 1] = fmaf(st.O[db][4 * j + 1], alpha, pr * hi_bf16(v.x));
          st.O[db][4 * j + 2] = fmaf(st.O[db][4 * j + 2], alpha, pr * lo_bf16(v.y));
          st.O[db][4 * j + 3] = fmaf(st.O[db][4 * j + 3], alpha, pr * hi_bf16(v.y));
        }
      }
    }
  }

  const int64_t n_rows_all = (int64_t)p.R * BW * p.Hq;
  const int64_t ri = qoff / D;
  // Debug variant: the Unshared partial is kept on its own (mu, lu, Ou),
  // written as stage 1, and the running state restarts for the Shared stage.
  float mu = -INFINITY, lu = 0.f;
  f32x16 Ou[TAPS ? NDB : 1];
  if constexpr (TAPS) {
    mu = st.m;
    lu = st.l;
    if (kh == 0) {
      const float inv = 1.f / st.l;
#pragma unroll
      for (int db = 0; db < NDB; ++db) Ou[db] = st.O[db] * inv;
      if (valid) {
        if (p.stage_ml && hl == 0) {
          p.stage_ml[(n_rows_all + ri) * 2 + 0] = st.m * p.scale;
          p.stage_ml[(n_rows_all + ri) * 2 + 1] = st.l;
        }
        if (p.stage_o) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              p.stage_o[(n_rows_all + ri) * D + db * 32 + 8 * (e / 4) + 4 * hl + e % 4] = Ou[db][e];
        }
      }
    }
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.O[db] = f32x16{};
  } else {
    // Seeded state: both lanes of a pair hold the full unshared sum; keep it
    // in one lane so the final pair-sum counts it once.
    st.l = hl == 0 ? st.l : 0.f;
  }

  // ---- Shared stage.  Tile `it` sits in stage it % NSTAGE.  Before
  // consuming it, every wave waits for its own copies of that tile (the
  // copies of the NSTAGE-2 later tiles may stay in flight) and the
  // workgroup synchronises; then the copy of tile it + NSTAGE - 1 goes into
  // the stage consumed in the previous iteration.
#define XATTN_STAGE(S) ((S) == 0 ? stage0 : ((S) == 1 ? stage1 : ((S) == 2 ? stage2 : stage3)))
#define XATTN_TILE_STEP(ST)                                                        \
  {                                                                                \
    const int it = it0 + (ST);                                                     \
    if (it >= n_tiles) break;                                                      \
    if (it + NSTAGE - 2 < n_tiles)                                                 \
      wait_vm_lgkm0<(NSTAGE - 2) * COPIES_PER_WAVE>();                             \
    else                                                                           \
      wait_vm_lgkm0<0>();                                                          \
    lds_barrier();                                                                 \
    if (it + NSTAGE - 1 < n_tiles)                                                 \
      tile_copy<D, WAVES>(XATTN_STAGE(((ST) + NSTAGE - 1) % NSTAGE), skg, svg,     \
                          (it + NSTAGE - 1) * KT, L, wave, lane);                  \
    consume_tile<D, KSPLIT>(XATTN_STAGE(ST), qf, st, kh, it * KT, L, c, thr, lane); \
  }
  static_assert(NSTAGE == 4, "the tile loop below is unrolled for 4 stages");
  for (int it0 = 0; it0 < n_tiles; it0 += NSTAGE) {
    XATTN_TILE_STEP(0)
    XATTN_TILE_STEP(1)
    XATTN_TILE_STEP(2)
    XATTN_TILE_STEP(3)
  }
#undef XATTN_TILE_STEP

  // ---- the second key half hands its state to the first through LDS
  // (stage buffer rg holds row group rg's exchange)
  if constexpr (KSPLIT == 2) {
    static_assert(RG <= NSTAGE, "one stage buffer per row group");
    static_assert((NDB * 16 + 2) * 64 * 4 <= Gm::STAGE_BYTES, "exchange must fit a stage");
    wait_vm_lgkm0<0>();
    lds_barrier();  // every wave is done with the tile stages
    float *xo = reinterpret_cast<float *>(XATTN_STAGE(rg));
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xo[(db * 16 + e) * 64 + lane] = st.O[db][e];
      xo[(NDB * 16) * 64 + lane] = st.m;
      xo[(NDB * 16 + 1) * 64 + lane] = st.l;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m2 = xo[(NDB * 16) * 64 + lane];
    const float l2 = xo[(NDB * 16 + 1) * 64 + lane];
    float a1 = 1.f, a2 = 0.f;
    if (m2 > st.m) {
      a1 = __builtin_amdgcn_exp2f((st.m - m2) * c);  // 0 when m is -inf
      a2 = 1.f;
      st.m = m2;
    } else if (m2 != -INFINITY) {
      a2 = __builtin_amdgcn_exp2f((m2 - st.m) * c);
    }
    st.l = st.l * a1 + l2 * a2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        st.O[db][e] = st.O[db][e] * a1 + xo[(db * 16 + e) * 64 + lane] * a2;
  }
#undef XATTN_STAGE

  // ---- Merge / epilogue
  const float lt = pair_sum(st.l);
  if constexpr (TAPS) {
    // Shared partial (m, lt, O / lt) on its own, then the explicit
    // OnlineSoftmax merge with the Unshared partial (mu, lu, Ou).
    const float ms = st.m;
    const float inv_s = lt > 0.f ? 1.f / lt : 0.f;
    const float mm = fmaxf(ms, mu);
    const float ws = lt > 0.f ? lt * __builtin_amdgcn_exp2f((ms - mm) * c) : 0.f;
    const float wu = lu * __builtin_amdgcn_exp2f((mu - mm) * c);
    const float inv_z = 1.f / (ws + wu);
    if (valid) {
      if (p.stage_ml && hl == 0) {
        p.stage_ml[ri * 2 + 0] = lt > 0.f ? ms * p.scale : -INFINITY;
        p.stage_ml[ri * 2 + 1] = lt;
      }
      if (p.stage_o) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            p.stage_o[ri * D + db * 32 + 8 * (e / 4) + 4 * hl + e % 4] = st.O[db][e] * inv_s;
      }
      if (p.lse && hl == 0) p.lse[ri] = mm * p.scale + __logf(ws + wu);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.O[db] = (st.O[db] * (inv_s * ws) + Ou[db] * wu) * inv_z;
  } else {
    const float inv = 1.f / lt;
    if (valid && p.lse && hl == 0) p.lse[ri] = st.m * p.scale + __logf(lt);
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.O[db] *= inv;
  }
  if (!valid) return;
  uint16_t *op = og + qoff;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x4 pk = {(__bf16)st.O[db][4 * j + 0], (__bf16)st.O[db][4 * j + 1],
                         (__bf16)st.O[db][4 * j + 2], (__bf16)st.O[db][4 * j + 3]};
      *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * j + 4 * hl) = pk;
    }
  }
}

template <int D, int RG, int KSPLIT, bool TAPS>
hipError_t launch_cfg(const DecodeParams &p0, hipStream_t stream) {
  constexpr int ROWS = RG * 32;
  DecodeParams p = p0;
  p.n_rb = (p.M + ROWS - 1) / ROWS;
  const int64_t grid = (int64_t)p.R * p.Hkv * p.n_rb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  size_t dyn = 0;
  if (p.anc == nullptr) {
    const int nb = min(p.BW, (ROWS - 1) / p.G + 2);
    dyn = (size_t)nb * (p.step + 1) * sizeof(int32_t);
  }
  hipLaunchKernelGGL((decode_bf16_kernel<D, RG, KSPLIT, TAPS>), dim3((unsigned)grid),
                     dim3(RG * KSPLIT * 64), dyn, stream, p);
  return hipGetLastError();
}

// Rows per workgroup: 32 (1 row group) or 64 (2) for few query rows per
// (request, KV head); otherwise 128 rows in 4 row groups.  Always two key
// halves.
int rows_per_block(int M) { return M <= 32 ? 32 : (M <= 64 ? 64 : 128); }

template <int D>
hipError_t launch_d(const DecodeParams &p, bool taps, hipStream_t stream) {
  const int rows = rows_per_block(p.M);
  if (taps) {
    if (rows == 32) return launch_cfg<D, 1, 2, true>(p, stream);
    if (rows == 64) return launch_cfg<D, 2, 2, true>(p, stream);
    return launch_cfg<D, 4, 2, true>(p, stream);
  }
  if (rows == 32) return launch_cfg<D, 1, 2, false>(p, stream);
  if (rows == 64) return launch_cfg<D, 2, 2, false>(p, stream);
  return launch_cfg<D, 4, 2, false>(p, stream);
}

}  // namespace

int bf16_rows_per_block(const DecodeParams &p) { return rows_per_block(p.M); }

hipError_t launch_decode_bf16(const DecodeParams &p, bool taps, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, taps, stream);
  if (p.D == 128) return launch_d<128>(p, taps, stream);
  return hipErrorInvalidValue;
}

}  // namespace xattn
