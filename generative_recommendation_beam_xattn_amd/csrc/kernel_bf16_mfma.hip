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
// Unshared stage: for chains of up to 16 levels, the generated-token rows
// of a row block are gathered into LDS in 32-row blocks laid out like the
// prompt tiles (TokenMap: row group g's tokens, beam-major and level-minor,
// each row copied from its beam's ancestor slot at its level).  The first
// block is copied right after the ancestor walk into a region of its own;
// the others go into ring stages the prompt stream has finished with.  Each
// block is contracted on the matrix cores like a 32-key prompt tile, with a
// block-diagonal mask so that a query row only sees its own beam's tokens,
// and enters the same online-softmax state: the Merge is that state's
// update.  Deeper chains, resolved into the workspace beforehand, are
// gathered from global memory by the lanes that hold the row (VALU dot
// products in fp32).  The debug variant (TAPS) keeps the two stages apart,
// writes each stage's (m, l, o) and merges them explicitly at the end.  Its
// two live states do not fit the registers at D = 128: the compiler spills
// inside the tile loops, and those scratch accesses count in vmcnt between
// the tile copies.  So every copy wait in that variant drains vmcnt to 0
// instead of leaving the newer tiles' copies in flight; the production
// variant keeps the pipelined counts.
#include <hip/hip_ext.h>

#include <algorithm>

#include "xattn_internal.h"

namespace xattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int KT = 64;      // keys per shared-stage tile
constexpr int NSTAGE = 4;   // LDS ring depth (tiles in flight = NSTAGE - 1)


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
// than p.lazy_log2 (kLazyRescaleLog2 = 8 on the decode path) in the exp2
// domain; until then p = exp2(s - m) may exceed 1 (by at most 256), which
// fp32 sums and bf16 P hold without loss of range.

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8) waiting for vmcnt <= VM and lgkmcnt == 0.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));
}

// LDS byte address of a generic pointer into LDS: its low 32 bits (the LDS
// aperture keeps the offset there).  Taken directly rather than through an
// address-space cast, whose null check the compiler has miscompiled here
// (an illegal compare against the shared aperture base).
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)p;
}

// One wave-wide 16-byte-per-lane copy global -> LDS (global_load_lds): lane
// i's 16 bytes at src land at LDS byte address lds_base + 16 i.  Issued as
// inline asm so that the compiler does not see the LDS write: it would
// otherwise put a full vmcnt(0) wait in front of LDS reads it cannot prove
// disjoint from copies in flight (the transposing V reads carry no alias
// information), draining the tile pipeline.  Every use of copied data is
// preceded by an explicit vmcnt wait and a barrier; the copy counts in vmcnt
// like any load, in issue order.
// NT: with the non-temporal hint (data no other workgroup reads soon).
// An LDS DMA that reads M0 in the instruction right after an M0 write is a
// hazard on this GPU family (one wait state is required, which the
// compiler inserts for its own code but cannot see inside asm): each block
// puts an s_nop between the two.
template <bool NT = true>
__device__ __forceinline__ void dma16(const void *src, const void *lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(lds_dst));
  uint32_t saved;  // M0 is the compiler's: put it back
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base)
        : "memory");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the instruction's saddr form): no per-lane 64-bit address
// arithmetic on the vector ALUs.
template <bool NT = true>
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, const void *lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(lds_dst));
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(base)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(base)
        : "memory");
}

// The same for 4 bytes per lane (global_load_lds_dword): lane i's 4 bytes
// at src land at LDS byte address lds_base + 4 i.
__device__ __forceinline__ void dma4(const void *src, const void *lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(lds_dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}

// Workgroup barrier that also orders this wave's LDS accesses in the
// compiler, without the vmcnt(0) a full fence would impose on the tile
// copies still in flight.  Callers wait for the copies they need first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Geometry of the LDS tiles: per stage a K tile and a V tile (separate
// LDS objects), each KTILE rows of D bf16, row-major, with the 16-byte
// slots of row r permuted by swz(r).
template <int D, int KTILE = KT>
struct TileGeom {
  static constexpr int RB = D * 2;                 // bytes per row
  static constexpr int SLOTS = D / 8;              // 16-byte slots per row
  static constexpr int TILE_BYTES = KTILE * RB;    // one K (or V) tile
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

// Distance from a ring stage's K tile to its V tile (the V tiles of all
// stages follow the K tiles of all stages).
template <int D, int KTILE = KT, int NST = NSTAGE>
__host__ __device__ constexpr int kVRegionOffset() { return NST * TileGeom<D, KTILE>::TILE_BYTES; }

// This wave's share of the COPIES wave-wide copies that fill one stage:
// copy i moves 1 KiB = ROWS_PER_COPY rows of the K tile (first NQ copies)
// or of the V tile.  Lane `lane` fetches row q * ROWS_PER_COPY + lane /
// SLOTS, 16-byte chunk (lane % SLOTS) ^ swz(row), which lands in LDS slot
// lane % SLOTS of that row.
template <int D, int WAVES, int KTILE = KT>
struct CopyPlan {
  using Gm = TileGeom<D, KTILE>;
  static constexpr int NQ = Gm::TILE_BYTES / 1024;   // copies per K (or V) tile
  static constexpr int PER = Gm::COPIES / WAVES;
  static_assert(Gm::COPIES % WAVES == 0, "copies must split evenly over the waves");
  uint32_t off[PER];   // byte offset of this lane's 16-byte chunk from the tile's first row
  __device__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int qi = wave * PER + i;
      const int q = qi >= NQ ? qi - NQ : qi;
      const int row = q * Gm::ROWS_PER_COPY + lane / Gm::SLOTS;
      off[i] = (uint32_t)(row * Gm::RB + (((lane % Gm::SLOTS) ^ Gm::swz(row)) << 4));
    }
  }
  __device__ static int row_of(uint32_t off) { return (int)(off / Gm::RB); }
};

// Copy the KT key rows starting at key0 into one ring stage (ktile, vtile).
// The caller keeps key0 + KT <= L whenever L >= KT (the last window is
// shifted back to end at L), so only a prompt shorter than one tile needs
// its rows clamped to the last one; clamped rows are always in bounds and
// their scores are masked.
template <int D, int WAVES, bool CLAMP, bool NT = true, int KTILE = KT>
__device__ __forceinline__ void tile_copy(uint8_t *ktile, uint8_t *vtile,
                                          const CopyPlan<D, WAVES, KTILE> &cp, const uint16_t *skg,
                                          const uint16_t *svg, int key0, int L, int wave) {
  using Gm = TileGeom<D, KTILE>;
  using C = CopyPlan<D, WAVES, KTILE>;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int qi = wave * C::PER + i;
    const bool is_v = qi >= C::NQ;
    const int q = is_v ? qi - C::NQ : qi;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(is_v ? svg : skg);
    uint8_t *dst = (is_v ? vtile : ktile) + q * 1024;
    if constexpr (!CLAMP) {
      // the tile's first row is uniform: only the lane's offset is per lane
      dma16s<NT>(base + (int64_t)key0 * Gm::RB, cp.off[i], dst);
    } else {
      const int row = C::row_of(cp.off[i]);
      const int key = min(key0 + row, L - 1);
      dma16<NT>(base + (int64_t)key * Gm::RB + (cp.off[i] - (uint32_t)(row * Gm::RB)), dst);
    }
  }
}

// Per-lane state of one wave's 32 query rows: running max m (raw dot-product
// units), O^T accumulators for this lane's 64 dims, and l, the sum of
// exp2((score - m) * c) over the keys this lane-pair has seen, split between
// the two lanes of the pair (the row total is pair_sum(l)).
template <int D>
struct Rows {
  float m, l;
  f32x16 O[D / 32];
  __device__ void clear() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) O[db] = f32x16{};
  }
};

// Per-lane LDS byte offsets of the MFMA A-operand fragments within a tile.
// K (ds_read_b128): row kh*NKB*32 + 32*i + ql, 16-byte slot (2ks + hl) ^
// swz(ql) -- the block index i only adds a multiple of 32 rows, so it is an
// immediate.  V^T (ds_read_b64_tr_b16): for k-step ps, half e2 and O block
// db the row is 32*(ps/2) + 16*(ps%2) + 8*e2 + 4h + j/4 and the slot
// (4db + 2g + (j/2)%2) ^ swz(row); swz(row) depends only on the lane and e2
// (the ps terms are multiples of 16 rows), so ps is an immediate as well.
template <int D, int VREG = kVRegionOffset<D>()>
struct FragOffsets {
  using Gm = TileGeom<D>;
  uint32_t k[D / 16];        // per ks
  uint32_t v[2][D / 32];     // per e2, db
  __device__ void init(int kh, int nkb, int lane) {
    const int hl = lane >> 5, ql = lane & 31;
    const int kswz = Gm::swz(ql);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      k[ks] = (uint32_t)((kh * nkb * 32 + ql) * Gm::RB + (((2 * ks + hl) ^ kswz) << 4));
    const int vh = lane >> 5, vg = (lane >> 4) & 1, vj = lane & 15;
    // the V offsets carry the key half's rows and the distance from the K
    // tiles to the V tiles of the ring, so that a V fragment's address is
    // (ring stage base + this register + an immediate below 64 KiB): the
    // V tiles themselves lie past the 16-bit offset field
    const int kv_region = VREG;
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int row = e2 * 8 + vh * 4 + (vj >> 2);   // plus multiples of 16
      const int sw = Gm::swz(row);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int chunk = 4 * db + 2 * vg + ((vj >> 1) & 1);
        v[e2][db] = (uint32_t)(kv_region + (kh * nkb * 32 + row) * Gm::RB + ((chunk ^ sw) << 4) +
                               ((vj & 1) << 3));
      }
    }
  }
};

// S^T = K . Q^T for this wave's 32-key block(s) of the tile in `ktile`.
template <int D, int KSPLIT, int VREG = kVRegionOffset<D>()>
__device__ __forceinline__ void qk_tile(const uint8_t *ktile, const bf16x8 (&qf)[D / 16],
                                        f32x16 (&sacc)[2 / KSPLIT], const FragOffsets<D, VREG> &fo) {
  using Gm = TileGeom<D>;
  constexpr int NKS = D / 16, NKB = 2 / KSPLIT;
#pragma unroll
  for (int i = 0; i < NKB; ++i) sacc[i] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int i = 0; i < NKB; ++i) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8 *>(ktile + fo.k[ks] + i * 32 * Gm::RB);
      sacc[i] = mfma(a, qf[ks], sacc[i]);
    }
  }
}

// Online-softmax update with one tile's scores, part 1: with TAIL, mask
// the keys outside [lo, L) (the tile holds keys key0 ..); take the row
// maximum and raise m lazily (rescaling l and O when it moves).  Returns
// m * c, the exp2 offset of part 2.
template <int D, int KSPLIT, bool TAIL>
__device__ __forceinline__ float softmax_max(f32x16 (&sacc)[2 / KSPLIT], Rows<D> &st, int kh,
                                             int key0, int lo, int L, float c, float thr,
                                             int lane) {
  constexpr int NDB = D / 32, NKB = 2 / KSPLIT;
  const int hl = lane >> 5;
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NKB; ++i) {
    const int kb = kh * NKB + i;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (TAIL) {
        const int key = key0 + kb * 32 + 8 * (e / 4) + 4 * hl + (e % 4);
        if (key < lo || key >= L) sacc[i][e] = -INFINITY;
      }
      tmax = fmaxf(tmax, sacc[i][e]);
    }
  }
  tmax = pair_max(tmax);
  if (__any(tmax > st.m + thr)) {
    // masks may differ between rows (token blocks): a row that has seen no
    // key yet and sees none here keeps m = -inf and its zero state
    const float mn = fmaxf(st.m, tmax);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((st.m - mn) * c);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.O[db] *= alpha;
  }
  // a key half can see only masked keys: m stays -inf and p = 0
  return st.m == -INFINITY ? 0.f : st.m * c;
}

// Part 1 for a tile whose row maxima were already taken (tmax: this lane's
// maximum over its scores of the tile, no masking): combine the lane pair
// and raise m lazily.  Returns m * c, as softmax_max.
template <int D>
__device__ __forceinline__ float softmax_max_finish(float tmax, Rows<D> &st, float c, float thr) {
  constexpr int NDB = D / 32;
  tmax = pair_max(tmax);
  if (__any(tmax > st.m + thr)) {
    const float mn = fmaxf(st.m, tmax);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((st.m - mn) * c);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.O[db] *= alpha;
  }
  return st.m == -INFINITY ? 0.f : st.m * c;
}

// Part 2 (branch-free): probabilities exp2(s * c - mc) as bf16 (the B
// operand of the PV product) and their sum into l, two per
// v_dot2_f32_bf16 against (1, 1), so l sums exactly the values PV uses.
template <int D, int KSPLIT>
__device__ __forceinline__ void softmax_exp(f32x16 (&sacc)[2 / KSPLIT], bf16x8 (&pf)[4 / KSPLIT],
                                            Rows<D> &st, float c, float mc) {
  constexpr int NKB = 2 / KSPLIT;
#pragma unroll
  for (int i = 0; i < NKB; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[i][e] = __builtin_amdgcn_exp2f(fmaf(sacc[i][e], c, -mc));
    pf[2 * i] = to_bf16x8(sacc[i], 0);
    pf[2 * i + 1] = to_bf16x8(sacc[i], 8);
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int j = 0; j < 2 * NKB; ++j) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pr = {pf[j][e], pf[j][e + 1]};
      st.l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, st.l, false);
    }
  }
}

// LDS fragment reads kept in flight ahead of the MFMA that consumes them: an
// LDS read takes longer than one MFMA plus its share of VALU work, so with
// one read ahead every MFMA waited on it.
constexpr int kFragAhead = 2;

// The S^T MFMAs of the next tile interleaved, k-step by k-step, with part 2
// of the current tile's softmax: each k-step issues the read of the K
// fragment kFragAhead steps on, its MFMA(s) and then a share of the
// exponentials, their bf16 packing and row sum, so the VALU works while the
// matrix core runs.  sched_barrier fences keep that order through
// scheduling.
template <int D, int KSPLIT, int VREG = kVRegionOffset<D>()>
__device__ __forceinline__ void qk_next_with_exp(const uint8_t *ktile, const bf16x8 (&qf)[D / 16],
                                                 f32x16 (&s_next)[2 / KSPLIT],
                                                 f32x16 (&s_cur)[2 / KSPLIT],
                                                 bf16x8 (&pf)[4 / KSPLIT], Rows<D> &st, float c,
                                                 float mc, const FragOffsets<D, VREG> &fo) {
  using Gm = TileGeom<D>;
  constexpr int NKS = D / 16, NKB = 2 / KSPLIT;
  constexpr int NV = 16 * NKB;        // scores per lane
  constexpr int PER = NV / NKS;       // exponentials per k-step (even)
  static_assert(PER % 2 == 0, "scores are packed in pairs");
#pragma unroll
  for (int i = 0; i < NKB; ++i) s_next[i] = f32x16{};
  bf16x8 a[NKS][NKB];   // indexed by unrolled constants only: registers
#pragma unroll
  for (int j = 0; j < kFragAhead && j < NKS; ++j)
#pragma unroll
    for (int i = 0; i < NKB; ++i)
      a[j][i] = *reinterpret_cast<const bf16x8 *>(ktile + fo.k[j] + i * 32 * Gm::RB);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks + kFragAhead < NKS) {
#pragma unroll
      for (int i = 0; i < NKB; ++i)
        a[ks + kFragAhead][i] =
            *reinterpret_cast<const bf16x8 *>(ktile + fo.k[ks + kFragAhead] + i * 32 * Gm::RB);
    }
#pragma unroll
    for (int i = 0; i < NKB; ++i) s_next[i] = mfma(a[ks][i], qf[ks], s_next[i]);
#pragma unroll
    for (int u = 0; u < PER; u += 2) {
      const int v = ks * PER + u;      // score index: block v / 16, element v % 16
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cur[v >> 4][v & 15], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cur[v >> 4][(v + 1) & 15], c, -mc));
      const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
      pf[v >> 3][v & 7] = pk[0];
      pf[v >> 3][(v + 1) & 7] = pk[1];
      // the row sum, issued here under the MFMA (as a plain intrinsic the
      // IR passes sink the whole chain to the step's end, where nothing
      // hides it): l += 1 * p0 + 1 * p1 on the packed pair
      asm volatile("v_dot2c_f32_bf16 %0, 0x3f803f80, %1"
                   : "+v"(st.l)
                   : "v"(__builtin_bit_cast(uint32_t, pk)));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T . P^T over this wave's keys of the tile in `vt`.  For k-step
// ps (16 keys) the B operand of lane half h holds the keys 32*(ps/2) +
// 16*(ps%2) + 8*e2 + 4h + (0..3), e2 = 0, 1; each half-fragment of V^T is one
// transposing read: lane j of a 16-lane group points at 4 dims of key row
// base + j/4, and receives 4 keys of dim d0 + (lane % 16).
template <int D, int KSPLIT, int VREG = kVRegionOffset<D>()>
__device__ __forceinline__ void pv_tile(const uint8_t *vt, const bf16x8 (&pf)[4 / KSPLIT],
                                        Rows<D> &st, int kh, const FragOffsets<D, VREG> &fo) {
  using Gm = TileGeom<D>;
  constexpr int NDB = D / 32, NKB = 2 / KSPLIT;
  const uint8_t *vbase = vt - VREG;   // fo.v holds the rest (and kh's rows)
  constexpr int NSTEP = 2 * NKB * NDB;
  // fragment n: k-step j2 = n / NDB (rows 32*(j2/2) + 16*(j2%2)), block db = n % NDB
  auto frag = [&](int n) {
    const int j2 = n / NDB, db = n % NDB;
    const int prow = (j2 >> 1) * 32 + (j2 & 1) * 16;
    const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(vbase + fo.v[0][db] + prow * Gm::RB));
    const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(vbase + fo.v[1][db] + prow * Gm::RB));
    return bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  };
  bf16x8 a[NSTEP];   // indexed by unrolled constants only: registers
#pragma unroll
  for (int j = 0; j < kFragAhead && j < NSTEP; ++j) a[j] = frag(j);
#pragma unroll
  for (int n = 0; n < NSTEP; ++n) {
    if (n + kFragAhead < NSTEP) a[n + kFragAhead] = frag(n + kFragAhead);
    st.O[n % NDB] = mfma(a[n], pf[n / NDB], st.O[n % NDB]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// pv_tile with the next tile's row maxima taken between its MFMAs: this
// lane's maximum over s_next (no masking) into tmax, one max3 per k-step
// from the second on, so the VALU works while the matrix core runs and the
// next step starts with only the lane-pair exchange left.
template <int D, int KSPLIT, int VREG = kVRegionOffset<D>()>
__device__ __forceinline__ void pv_tile_max(const uint8_t *vt, const bf16x8 (&pf)[4 / KSPLIT],
                                            Rows<D> &st, int kh, const FragOffsets<D, VREG> &fo,
                                            const f32x16 (&s_next)[2 / KSPLIT], float &tmax) {
  using Gm = TileGeom<D>;
  constexpr int NDB = D / 32, NKB = 2 / KSPLIT;
  const uint8_t *vbase = vt - VREG;   // fo.v holds the rest (and kh's rows)
  constexpr int NSTEP = 2 * NKB * NDB;
  constexpr int NV = 16 * NKB;                      // scores per lane
  // scores per k-step (steps 1..NSTEP-1), even: two per v_max3_f32
  constexpr int PER = ((NV + NSTEP - 2) / (NSTEP - 1) + 1) & ~1;
  static_assert(NSTEP >= 2, "maxima start at the second k-step");
  auto frag = [&](int n) {
    const int j2 = n / NDB, db = n % NDB;
    const int prow = (j2 >> 1) * 32 + (j2 & 1) * 16;
    const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(vbase + fo.v[0][db] + prow * Gm::RB));
    const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(vbase + fo.v[1][db] + prow * Gm::RB));
    return bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  };
  bf16x8 a[NSTEP];
#pragma unroll
  for (int j = 0; j < kFragAhead && j < NSTEP; ++j) a[j] = frag(j);
  tmax = -INFINITY;
#pragma unroll
  for (int n = 0; n < NSTEP; ++n) {
    if (n + kFragAhead < NSTEP) a[n + kFragAhead] = frag(n + kFragAhead);
    st.O[n % NDB] = mfma(a[n], pf[n / NDB], st.O[n % NDB]);
    if (n >= 1 && (n - 1) * PER < NV) {
      // two scores per v_max3_f32, issued here: as plain fmaxf the IR passes
      // sink the pure max chain past the scheduling fence to its use, and a
      // chain broken at each step costs a quieting max per operand (scores
      // are finite or -inf, never NaN, so the ordering of v_max3 is exact)
#pragma unroll
      for (int u = 0; u < PER; u += 2) {
        const int v = (n - 1) * PER + u;
        if (v + 1 < NV) {
          asm volatile("v_max3_f32 %0, %0, %1, %2"
                       : "+v"(tmax)
                       : "v"(s_next[v >> 4][v & 15]), "v"(s_next[(v + 1) >> 4][(v + 1) & 15]));
        } else if (v < NV) {
          asm volatile("v_max_f32 %0, %0, %1" : "+v"(tmax) : "v"(s_next[v >> 4][v & 15]));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Generated-token rows of a row block, gathered into LDS in the layout of
// the prompt tiles, in blocks of 32 rows.  Row group g of the block has
// n_blk blocks; block b of it holds its tokens 32 b .. 32 b + 31, token i
// being (beam first(g) + i / nlev, level i % nlev), nlev = step + 1, where
// first(g) is the beam of the group's first query row.  Blocks are
// numbered gb = b * RG + g.  A row's source is the token row of its beam's
// ancestor slot at its level (anc_lds [nb][step + 1], indexed from the row
// block's first beam b_lo); rows past a group's tokens repeat a valid row
// (their scores are masked).
template <int RG>
struct TokenMap {
  const int32_t *anc_lds;
  int n_blk, nlev, BW, nb;
  // i / nlev == (i * nlev_magic) >> 20 for the token counts used here
  // (i * nlev < 2^20), nlev_magic = floor(2^20 / nlev) + 1
  uint32_t nlev_magic;
  // first beam of row group g, from the row block's first beam:
  // (row0 + 32 g) / G - b_lo, which is first0 + g * gstep when G divides 32
  // (a scalar formula: an array indexed by g would live in scratch memory)
  int first0, gstep, G, row0, b_lo;
  bool linear;
  __device__ void init(const int32_t *anc, int n_blk_, int nlev_, int BW_, int nb_, int G_,
                       int row0_, int b_lo_) {
    anc_lds = anc;
    n_blk = n_blk_;
    nlev = nlev_;
    BW = BW_;
    nb = nb_;
    nlev_magic = (1u << 20) / (uint32_t)nlev_ + 1u;
    G = G_;
    row0 = row0_;
    b_lo = b_lo_;
    linear = 32 % G_ == 0;
    first0 = row0_ / G_ - b_lo_;
    gstep = linear ? 32 / G_ : 0;
  }
  __device__ int first(int g) const {
    return linear ? first0 + g * gstep : (row0 + 32 * g) / G - b_lo;
  }
  // row index (level * BW + slot) of row r of block gb in the (request, KV
  // head) slice of the unshared cache
  __device__ int row_index(int gb, int r) const {
    gb = min(gb, RG * n_blk - 1);
    const int g = gb % RG, b = gb / RG;
    const int i = 32 * b + r;
    const int jb = (int)(((uint32_t)i * nlev_magic) >> 20);
    const int lvl = i - jb * nlev;
    const int bi = clampi(first(g) + jb, 0, nb - 1);
    return lvl * BW + anc_lds[bi * nlev + lvl];
  }
  // element offset of row r of block gb in the (request, KV head) slice
  __device__ int64_t row_elem(int gb, int r, int D) const {
    gb = min(gb, RG * n_blk - 1);
    const int g = gb % RG, b = gb / RG;
    const int i = 32 * b + r;
    const int jb = (int)(((uint32_t)i * nlev_magic) >> 20);
    const int lvl = i - jb * nlev;
    const int bi = clampi(first(g) + jb, 0, nb - 1);
    const int slot = anc_lds[bi * nlev + lvl];
    return ((int64_t)lvl * BW + slot) * D;
  }
};

// Blocks 1 + 2c and 2 + 2c as one KT-row tile (chunk c), with the prompt
// tiles' copy plan; rows[i] is the row index of copy i's row (TokenMap::
// row_index), read from registers so that no LDS read sits between the
// copies in flight and this one.
template <int D, int WAVES>
__device__ __forceinline__ void token_chunk_copy_rows(uint8_t *ktile, uint8_t *vtile,
                                                      const CopyPlan<D, WAVES> &cp,
                                                      const uint16_t *ukg, const uint16_t *uvg,
                                                      const int (&rows)[CopyPlan<D, WAVES>::PER],
                                                      int wave) {
  using Gm = TileGeom<D>;
  using C = CopyPlan<D, WAVES>;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int qi = wave * C::PER + i;
    const bool is_v = qi >= C::NQ;
    const int q = is_v ? qi - C::NQ : qi;
    const int row = C::row_of(cp.off[i]);
    const uint8_t *src = reinterpret_cast<const uint8_t *>((is_v ? uvg : ukg) + (int64_t)rows[i] * D) +
                         (cp.off[i] - (uint32_t)(row * Gm::RB));
    dma16(src, ((is_v ? vtile : ktile) + q * 1024));
  }
}

// Blocks 1 + 2c and 2 + 2c as one KT-row tile (chunk c), with the prompt
// tiles' copy plan.
template <int D, int WAVES, int RG>
__device__ __forceinline__ void token_chunk_copy(uint8_t *ktile, uint8_t *vtile,
                                                 const CopyPlan<D, WAVES> &cp,
                                                 const uint16_t *ukg, const uint16_t *uvg,
                                                 const TokenMap<RG> &tm, int chunk, int wave) {
  using Gm = TileGeom<D>;
  using C = CopyPlan<D, WAVES>;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int qi = wave * C::PER + i;
    const bool is_v = qi >= C::NQ;
    const int q = is_v ? qi - C::NQ : qi;
    const int row = C::row_of(cp.off[i]);
    const int64_t e = tm.row_elem(1 + 2 * chunk + row / 32, row % 32, D);
    const uint8_t *src = reinterpret_cast<const uint8_t *>((is_v ? uvg : ukg) + e) +
                         (cp.off[i] - (uint32_t)(row * Gm::RB));
    dma16(src, ((is_v ? vtile : ktile) + q * 1024));
  }
}

// Wave-wide copies per wave that token_block0_copy issues.
template <int D, int WAVES>
constexpr int block0_copies_per_wave() { return 2 * (32 * TileGeom<D>::RB / 1024) / WAVES; }

// Block 0 into its own region (32 rows of K at sk, of V at sv).
template <int D, int WAVES, int RG>
__device__ __forceinline__ void token_block0_copy(uint8_t *sk, uint8_t *sv, const uint16_t *ukg,
                                                  const uint16_t *uvg, const TokenMap<RG> &tm,
                                                  int wave, int lane) {
  using Gm = TileGeom<D>;
  constexpr int NQ = 32 * Gm::RB / 1024;  // 1 KiB copies per K (or V) block
  static_assert((2 * NQ) % WAVES == 0, "block copies must split evenly over the waves");
  constexpr int PER = 2 * NQ / WAVES;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int qi = wave * PER + i;
    const bool is_v = qi >= NQ;
    const int q = is_v ? qi - NQ : qi;
    const int row = q * Gm::ROWS_PER_COPY + lane / Gm::SLOTS;
    const int64_t e = tm.row_elem(0, row, D);
    const uint8_t *src = reinterpret_cast<const uint8_t *>((is_v ? uvg : ukg) + e) +
                         (((lane % Gm::SLOTS) ^ Gm::swz(row)) << 4);
    dma16(src, ((is_v ? sv : sk) + q * 1024));
  }
}

// Unshared stage on the matrix cores: one token block (rows at kt / vt, K
// and V) against the wave's 32 query rows, as a 32-key tile whose scores
// are masked block-diagonally: token i0 + i counts for a query row iff it
// lies in [tok_lo, tok_hi), the row's own tokens (its beam's levels).
template <int D, int KSPLIT, int VREG = kVRegionOffset<D>()>
__device__ __forceinline__ void token_block(Rows<D> &st, const bf16x8 (&qf)[D / 16],
                                            const uint8_t *kt, const uint8_t *vt,
                                            const FragOffsets<D, VREG> &fo, int kh, int i0, int tok_lo,
                                            int tok_hi, float c, float thr, int lane) {
  static_assert(KSPLIT == 2, "a token block is one 32-key block per wave");
  using Gm = TileGeom<D>;
  const int hl = lane >> 5;
  // the fragment offsets carry the key half's row offset: cancel it
  const uint8_t *kb = kt - kh * 32 * Gm::RB;
  const uint8_t *vb = vt - kh * 32 * Gm::RB;
  f32x16 sb[1];
  qk_tile<D, KSPLIT, VREG>(kb, qf, sb, fo);
  const int base = i0 + 4 * hl - tok_lo;
  const uint32_t span = (uint32_t)max(tok_hi - tok_lo, 0);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t d = (uint32_t)(base + 8 * (e / 4) + (e % 4));
    sb[0][e] = d < span ? sb[0][e] : -INFINITY;
  }
  bf16x8 pf[2];
  const float mc = softmax_max<D, KSPLIT, false>(sb, st, kh, 0, 0, 0, c, thr, lane);
  softmax_exp<D, KSPLIT>(sb, pf, st, c, mc);
  pv_tile<D, KSPLIT, VREG>(vb, pf, st, kh, fo);
}

// Online-softmax state of query row `ri` from the Unshared-stage partial
// (m, l, unnormalised o) written by the token-partials kernel: l goes to lane
// half 0 (a row's l is the sum over the lane pair).
template <int D>
__device__ __forceinline__ void seed_rows(Rows<D> &s, const DecodeParams &p, int64_t ri, int hl) {
  s.m = p.tok_ml[ri * 2 + 0];
  s.l = hl == 0 ? p.tok_ml[ri * 2 + 1] : 0.f;
  const float *po = p.tok_o + ri * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4 *>(po + db * 32 + 8 * j + 4 * hl);
      s.O[db][4 * j + 0] = v.x;
      s.O[db][4 * j + 1] = v.y;
      s.O[db][4 * j + 2] = v.z;
      s.O[db][4 * j + 3] = v.w;
    }
}

// Key half 1 of a row group hands its state to key half 0 through LDS (xo:
// O, 16 bytes per lane and step; xs: m, then l), and key half 0 folds it in.
template <int D>
__device__ __forceinline__ void half_put(const Rows<D> &s, float4 *xo, float *xs, int lane) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xo[(db * 4 + j) * 64 + lane] =
          make_float4(s.O[db][4 * j], s.O[db][4 * j + 1], s.O[db][4 * j + 2], s.O[db][4 * j + 3]);
  xs[lane] = s.m;
  xs[64 + lane] = s.l;
}

template <int D>
__device__ __forceinline__ void half_merge(Rows<D> &s, const float4 *xo, const float *xs, float c,
                                           int lane) {
  const float m2 = xs[lane];
  const float l2 = xs[64 + lane];
  float a1 = 1.f, a2 = 0.f;
  if (m2 > s.m) {
    a1 = __builtin_amdgcn_exp2f((s.m - m2) * c);  // 0 when m is -inf
    a2 = 1.f;
    s.m = m2;
  } else if (m2 != -INFINITY) {
    a2 = __builtin_amdgcn_exp2f((m2 - s.m) * c);
  }
  s.l = s.l * a1 + l2 * a2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 o2 = xo[(db * 4 + j) * 64 + lane];
      s.O[db][4 * j + 0] = s.O[db][4 * j + 0] * a1 + o2.x * a2;
      s.O[db][4 * j + 1] = s.O[db][4 * j + 1] * a1 + o2.y * a2;
      s.O[db][4 * j + 2] = s.O[db][4 * j + 2] * a1 + o2.z * a2;
      s.O[db][4 * j + 3] = s.O[db][4 * j + 3] * a1 + o2.w * a2;
    }
}

// Parent rows of levels 1..step are copied to LDS for the in-kernel walk
// when they hold at most this many ints and the workgroup's LDS allows.
constexpr int kParentLdsInts = 2048;

// Static LDS of the kernel: the tile ring (K tiles of all stages, then V
// tiles), then token block 0 (32 rows of K, then of V).
template <int D>
constexpr int kTilesLdsBytes = 2 * NSTAGE * TileGeom<D>::TILE_BYTES + 2 * 32 * TileGeom<D>::RB;

// Most beams the query rows of one workgroup belong to: row blocks start at
// multiples of `rows`, so when G divides `rows` a block holds rows / G whole
// beams; otherwise it may also hold part of a beam at either end.
int beams_per_block(int rows, int G, int BW) {
  const int nb = rows % G == 0 ? rows / G : (rows - 1) / G + 2;
  return std::min(nb, BW);
}

template <int D, int RG, int KSPLIT, bool TAPS>
__global__ __launch_bounds__(RG * KSPLIT * 64) void decode_bf16_kernel(DecodeParams p) {
  constexpr int WAVES = RG * KSPLIT;
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = RG * 32;
  constexpr int NKS = D / 16;           // k-steps of the QK contraction
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int NKB = 2 / KSPLIT;       // 32-key blocks per wave per tile
  using Gm = TileGeom<D>;
  constexpr int CPW = Gm::COPIES / WAVES;   // wave-wide copies per wave per tile

  // The tile ring: K tiles of stages 0..3, then V tiles of stages 0..3, in
  // one LDS object at constant offsets.  Constant offsets let every
  // fragment address be a per-lane register plus an immediate, and let the
  // compiler see that a copy into one stage does not alias reads of
  // another (so it adds no wait of its own in front of those reads).
  // After the ring, token block 0 (32 rows of K, then of V).
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[kTilesLdsBytes<D>];
  // dynamic: ancestor slots [beams of the block][step + 1], then (when
  // staged) the parent rows [step][BW] of levels 1..step
  extern __shared__ int32_t dyn_lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int rg = wave % RG;     // row group
  const int kh = wave / RG;     // key half
  const int hl = lane >> 5;     // lane half
  const int ql = lane & 31;     // query (B/C column) of this lane

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rb = lb % p.n_rb;
  const int split = (lb / p.n_rb) % p.n_split;   // key split (row blocks of one split adjacent)
  const int unit = lb / p.n_rb / p.n_split;
  const int r = __builtin_amdgcn_readfirstlane(unit / p.Hkv);
  const int k = unit % p.Hkv;
  const int G = p.G, BW = p.BW, step = p.step;
  // the prompt length first, before any copy is issued: a scalar load whose
  // wait does not involve the vector-memory counter the copies run on
  const int L = clampi(p.prompt_len[r], 0, p.Lmax);
  const float c = p.scale_log2;
  // in raw dot-product units; the debug entry passes 0, so that the stages'
  // maxima it reports are the true ones
  const float thr = p.lazy_log2 / c;

  const int row0 = rb * ROWS;
  // the beams rows row0 .. row0 + ROWS - 1 (clipped to the M rows) belong to
  const int b_lo = row0 / G;
  const int nb = (min(row0 + ROWS, p.M) - 1) / G - b_lo + 1;
  int32_t *anc_lds = dyn_lds;
  int32_t *par_lds = dyn_lds + nb * (step + 1);
  const bool walk_here = p.anc == nullptr;
  const bool staged = walk_here && p.stage_par != 0;

  // ---- copies into LDS that depend on nothing, issued before the tile
  // copies (vmcnt counts in issue order, so the wait for tile 0 covers
  // them): the parent rows of levels 1..step for the walk, and the q rows of
  // each row group -- its key-half-0 wave copies them into ring stage 3,
  // which no tile uses before the first loop step, and both waves of the
  // group read them from there.  No vector load the compiler sees is in
  // flight, so it adds no wait of its own for them.
  const int32_t *par = p.parent_idx + (int64_t)r * p.S * BW;
  if (staged) {
    const int n_par = step * BW;
    for (int c0 = wave * 64; c0 < n_par; c0 += WAVES * 64)
      dma4(par + BW + min(c0 + lane, n_par - 1), par_lds + c0);
  }
  const uint16_t *qg = static_cast<const uint16_t *>(p.q);
  uint16_t *og = static_cast<uint16_t *>(p.out);
  const int row = row0 + rg * 32 + ql;
  const bool valid = row < p.M;
  const int rr = valid ? row : p.M - 1;
  const int beam = rr / G;
  const int64_t qoff = (((int64_t)r * BW + beam) * p.Hq + k * G + rr % G) * D;
  // stage 3 holds the q rows of row groups 0, 1 (K buffer) and 2, 3 (V
  // buffer): the group's 32 rows laid out like a tile's (row-major, 16-byte
  // slots permuted by swz), so that each copy reads ROWS_PER_COPY whole rows
  // and the fragment reads below are free of bank conflicts
  static_assert(32 * Gm::RB == NKS * 1024, "a row group's q rows are NKS 1 KiB copies");
  const uint8_t *qlds = tiles + ((rg < 2 ? 3 : NSTAGE + 3) * Gm::TILE_BYTES) +
                        (rg & 1) * (32 * Gm::RB);
  if (kh == 0) {
#pragma unroll
    for (int n = 0; n < NKS; ++n) {
      const int qr = n * Gm::ROWS_PER_COPY + lane / Gm::SLOTS;   // row of the group
      const int qrr = min(row0 + rg * 32 + qr, p.M - 1);
      const int qb = qrr / G;
      const int64_t qro = (((int64_t)r * BW + qb) * p.Hq + k * G + (qrr - qb * G)) * D;
      dma16<false>(qg + qro + (((lane % Gm::SLOTS) ^ Gm::swz(qr)) << 3), qlds + n * 1024);
    }
  }

  const uint16_t *ukg = static_cast<const uint16_t *>(p.unshared_k) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  const uint16_t *uvg = static_cast<const uint16_t *>(p.unshared_v) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;

  // ---- start the tile pipeline: tiles 0 .. NSTAGE-2 in flight.  When the
  // cache holds at least three tiles of rows, the copies of keys [0, 3 KT)
  // start at once, before the prompt length is known (rows at or past it
  // are allocated and are never counted); they are right whenever the
  // prompt has more than three tiles, and are redone otherwise.
  const uint16_t *skg = static_cast<const uint16_t *>(p.shared_k) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *svg = static_cast<const uint16_t *>(p.shared_v) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  CopyPlan<D, WAVES> cplan;
  cplan.init(wave, lane);
  const bool speculate = p.n_split == 1 && p.Lmax >= 3 * KT;
  if (speculate) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
      tile_copy<D, WAVES, false, false>(tiles + i * Gm::TILE_BYTES, tiles + (NSTAGE + i) * Gm::TILE_BYTES,
                                 cplan, skg, svg, i * KT, 0, wave);
  }
  // The prompt's tiles are split evenly over the key splits; this
  // workgroup takes tiles [t_base, t_base + n_tiles) (its tile t is prompt
  // tile t_base + t).
  const int n_tiles_all = (L + KT - 1) / KT;
  const int t_base = split * n_tiles_all / p.n_split;
  const int n_tiles = (split + 1) * n_tiles_all / p.n_split - t_base;
  // Prompt tile g covers keys [g*KT, g*KT + KT); the last one's window is
  // shifted back to [L - KT, L) (when L >= KT) so that no copy needs
  // clamping; its keys below g * KT were already counted and get masked.
  const int last_key0 = L >= KT ? L - KT : 0;
#define XATTN_KT(S) (tiles + (S) * Gm::TILE_BYTES)
#define XATTN_VT(S) (tiles + (NSTAGE + (S)) * Gm::TILE_BYTES)
#define XATTN_KEY0(T) (t_base + (T) + 1 < n_tiles_all ? (t_base + (T)) * KT : last_key0)
  if (speculate && n_tiles > 3) {
    // the speculative copies are tiles 0, 1, 2
  } else if (L < KT) {
    if (speculate) wait_vm_lgkm0<0>();  // this wave's copies into the stages have landed
    if (n_tiles > 0)
      tile_copy<D, WAVES, true, false>(XATTN_KT(0), XATTN_VT(0), cplan, skg, svg, 0, L, wave);
  } else {
    if (speculate) wait_vm_lgkm0<0>();
    tile_copy<D, WAVES, false, false>(XATTN_KT(0), XATTN_VT(0), cplan, skg, svg, XATTN_KEY0(0), L,
                                      wave);
    if (n_tiles > 1)
      tile_copy<D, WAVES, false, false>(XATTN_KT(1), XATTN_VT(1), cplan, skg, svg, XATTN_KEY0(1), L,
                                 wave);
    if (n_tiles > 2)
      tile_copy<D, WAVES, false, false>(XATTN_KT(2), XATTN_VT(2), cplan, skg, svg, XATTN_KEY0(2), L,
                                 wave);
  }

  // ---- generated-token rows.  With the ancestor slots in LDS they are
  // gathered into LDS in 32-row blocks (TokenMap): block 0 into a region of
  // its own as soon as the slots are known, blocks 1 + 2c and 2 + 2c as
  // chunk c, a KT-row tile.  Chunk c is copied at loop step chunk_t0 + c
  // into the stage that step frees, in the last two steps, where no prompt
  // tile remains to copy, so it lands while the last prompt tiles are
  // consumed; chunks that find no such step are copied after the loop.
  // Deep chains (slots in the workspace) get their Unshared stage from a
  // kernel run beforehand (below).
  const bool lds_tokens = walk_here;
  const int nlev = step + 1;
  const int nbr_max = (32 % G == 0) ? 32 / G : 32 / G + 2;  // beams 32 rows can touch
  const int n_blk = (nbr_max * nlev + 31) / 32;
  const int n_chunks = lds_tokens ? RG * n_blk / 2 : 0;
  const int chunk_t0 = max(0, n_tiles - 3);
  TokenMap<RG> tmap;
  tmap.init(anc_lds, n_blk, nlev, BW, nb, G, row0, b_lo);
#define XATTN_SK (tiles + 2 * NSTAGE * Gm::TILE_BYTES)
#define XATTN_SV (tiles + 2 * NSTAGE * Gm::TILE_BYTES + 32 * Gm::RB)

  constexpr int B0PW = block0_copies_per_wave<D, WAVES>();
  // rows of the two chunks the loop may copy (the last two steps), read
  // from LDS once the ancestor slots are in (two named arrays: an array
  // indexed by a runtime chunk number would live in scratch memory)
  int chunk_rows0[CopyPlan<D, WAVES>::PER], chunk_rows1[CopyPlan<D, WAVES>::PER];
// (macros, not lambdas: a lambda capturing the LDS ring turns its address
// into a generic pointer, and the cast back in the copies miscompiles)
#define XATTN_WALK()                                                                  \
  for (int i = tid; i < nb; i += NT) {                                                \
    int a = b_lo + i;                                                                 \
    int32_t *dst = anc_lds + i * (step + 1);                                          \
    dst[step] = a;                                                                    \
    for (int t = step; t >= 1; --t) {                                                 \
      a = clampi(staged ? par_lds[(t - 1) * BW + a] : par[(int64_t)t * BW + a], 0, BW - 1); \
      dst[t - 1] = a;                                                                 \
    }                                                                                 \
  }
#define XATTN_ISSUE_BLOCK0()                                                          \
  {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < CopyPlan<D, WAVES>::PER; ++i) {             \
      const int row = CopyPlan<D, WAVES>::row_of(cplan.off[i]);                       \
      chunk_rows0[i] = tmap.row_index(1 + row / 32, row % 32);                        \
      chunk_rows1[i] = tmap.row_index(3 + row / 32, row % 32);                        \
    }                                                                                 \
    token_block0_copy<D, WAVES>(XATTN_SK, XATTN_SV, ukg, uvg, tmap, wave, lane);      \
  }
  // On the common path (the first three tiles copied speculatively, parent
  // rows staged) the walk waits for the parent rows alone, the oldest
  // copies: it and the copy of token block 0 then run under the latency of
  // tile 0 instead of after it.  The wait leaves this wave's q copies
  // (key half 0) and its three tiles' copies in flight, which the vmcnt
  // field must be able to count.
  constexpr bool kEarlyWalkFits = 3 * CPW + NKS < 64;
  const bool early_walk = kEarlyWalkFits && staged && lds_tokens && speculate && n_tiles > 3;
  if (early_walk) {
    if constexpr (kEarlyWalkFits) {
      if (kh == 0)
        wait_vm_lgkm0<TAPS ? 0 : (3 * CPW + NKS)>();
      else
        wait_vm_lgkm0<TAPS ? 0 : (3 * CPW)>();
    }
    lds_barrier();   // every wave's parent copies have landed
    XATTN_WALK()
    lds_barrier();   // the ancestor slots are visible
    XATTN_ISSUE_BLOCK0()
    // tile 0 and q, older than tiles 1, 2 and block 0
    wait_vm_lgkm0<TAPS ? 0 : (2 * CPW + B0PW)>();
    lds_barrier();   // tile 0 and q are visible
  } else {
    // ---- wait for tile 0 (the parent rows and q are older, so they are in
    // too), then the ancestor slots of the block's beams (short chains:
    // walked here, from the parent rows staged in LDS)
    if (n_tiles > 2)
      wait_vm_lgkm0<TAPS ? 0 : (2 * CPW)>();
    else if (n_tiles > 1)
      wait_vm_lgkm0<TAPS ? 0 : CPW>();
    else
      wait_vm_lgkm0<0>();
    if (staged) lds_barrier();   // every wave's parent copies have landed
    if (walk_here) XATTN_WALK()
    lds_barrier();  // tile 0, q and the ancestor slots are visible
    if (lds_tokens) XATTN_ISSUE_BLOCK0()
  }
#undef XATTN_WALK
#undef XATTN_ISSUE_BLOCK0
  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8 *>(qlds + ql * Gm::RB +
                                                (((2 * ks + hl) ^ Gm::swz(ql)) << 4));

  // st: the online-softmax state of the row; with TAPS, of the Shared stage
  // alone, and su that of the Unshared stage (the debug entry keeps the
  // stages apart and merges them explicitly at the end)
  Rows<D> st, su;
  st.clear();
  su.clear();
  if (!walk_here) {
    // deep chains: the Unshared stage was computed beforehand, one workgroup
    // per (request, beam, KV head); key half 0 of key split 0 starts from its
    // partial (key half 1 starts empty; l lives in lane half 0, the row
    // total being the pair's sum)
    if (kh == 0 && split == 0) {
      if constexpr (TAPS)
        seed_rows<D>(su, p, qoff / D, hl);
      else
        seed_rows<D>(st, p, qoff / D, hl);
    }
    // the compiler counts these loads, not the tile copies issued before
    // them: left pending, they would make it wait for vmcnt to reach 0 at
    // their first use inside the tile loop, every iteration, draining the
    // copy pipeline; completing them here clears that for the whole loop
    wait_vm_lgkm0<0>();
  }

  // ---- Shared stage.  Per tile t (in stage t % NSTAGE) but the last: wait
  // for tile t + 1 and synchronise, finish the row maxima of tile t, then
  // issue the S^T MFMAs of tile t + 1 interleaved with the exponentials of
  // tile t (the matrix cores and the VALU work side by side), then tile t's
  // PV MFMAs, then copy tile t + 3 (or a token chunk) into the stage tile
  // t - 1 used.
  FragOffsets<D> fo;
  fo.init(kh, NKB, lane);
  f32x16 s_cur[NKB], s_next[NKB];
  bf16x8 pf[2 * NKB];
  if (n_tiles > 0) qk_tile<D, KSPLIT>(XATTN_KT(0), qf, s_cur, fo);
  // this lane's maximum over the scores of the tile the next loop step
  // consumes (loop tiles are never masked: only the last tile is)
  float tmax_cur = -INFINITY;
#pragma unroll
  for (int i = 0; i < NKB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) tmax_cur = fmaxf(tmax_cur, s_cur[i][e]);
// whether step u's end copied something (tile u + 3, or chunk u - chunk_t0;
// at most two chunks are copied in the loop)
#define XATTN_COPIED(u) \
  ((u) + 3 < n_tiles || ((u) >= chunk_t0 && (u) - chunk_t0 < n_chunks))
#define XATTN_TILE_STEP(ST)                                                           \
  {                                                                                   \
    const int t = t0 + (ST);                                                          \
    if (t + 1 >= n_tiles) break;                                                      \
    /* tile t + 1 is in once all but the copies younger than it are: the */        \
    /* copy of step t - 1 (tile t + 2 or a chunk), and for t < 2 the */              \
    /* prologue's tile 2 (t = 0) and block 0 */                                       \
    {                                                                                 \
      const bool cp_prev = t >= 1 && XATTN_COPIED(t - 1);                             \
      const bool cp_more = t == 0 && n_tiles > 2;                                     \
      const bool b0 = t < 2 && lds_tokens;                                            \
      const int units = (cp_prev ? 1 : 0) + (cp_more ? 1 : 0);                        \
      if (b0) {                                                                       \
        if (units == 0) wait_vm_lgkm0<TAPS ? 0 : B0PW>();                             \
        else wait_vm_lgkm0<TAPS ? 0 : (B0PW + CPW)>();                                \
      } else {                                                                        \
        if (units == 0) wait_vm_lgkm0<0>();                                           \
        else wait_vm_lgkm0<TAPS ? 0 : CPW>();                                         \
      }                                                                               \
    }                                                                                 \
    lds_barrier();                                                                    \
    const float mc = softmax_max_finish<D>(tmax_cur, st, c, thr);                     \
    qk_next_with_exp<D, KSPLIT>(XATTN_KT(((ST) + 1) % NSTAGE), qf, s_next, s_cur, pf, st, \
                                c, mc, fo);                                           \
    pv_tile_max<D, KSPLIT>(XATTN_VT(ST), pf, st, kh, fo, s_next, tmax_cur);           \
    if (t + 3 < n_tiles)                                                              \
      tile_copy<D, WAVES, false>(XATTN_KT(((ST) + 3) % NSTAGE),                       \
                                 XATTN_VT(((ST) + 3) % NSTAGE), cplan, skg, svg,      \
                                 XATTN_KEY0(t + 3), L, wave);                         \
    else if (XATTN_COPIED(t)) {                                                       \
      int rows_t[CopyPlan<D, WAVES>::PER];                                            \
      _Pragma("unroll") for (int i = 0; i < CopyPlan<D, WAVES>::PER; ++i)             \
        rows_t[i] = t > chunk_t0 ? chunk_rows1[i] : chunk_rows0[i];                   \
      token_chunk_copy_rows<D, WAVES>(XATTN_KT(((ST) + 3) % NSTAGE),                   \
                                      XATTN_VT(((ST) + 3) % NSTAGE), cplan, ukg, uvg,  \
                                      rows_t, wave);                                  \
    }                                                                                 \
    _Pragma("unroll") for (int i = 0; i < NKB; ++i) s_cur[i] = s_next[i];             \
  }
  static_assert(NSTAGE == 4, "the tile loop below is unrolled for 4 stages");
  for (int t0 = 0; t0 + 1 < n_tiles; t0 += NSTAGE) {
    XATTN_TILE_STEP(0)
    XATTN_TILE_STEP(1)
    XATTN_TILE_STEP(2)
    XATTN_TILE_STEP(3)
  }
#undef XATTN_TILE_STEP
#undef XATTN_COPIED
  if (n_tiles > 0) {  // the last tile: every copy has landed
    const int t = n_tiles - 1;
    const int lo = (t_base + t) * KT;   // keys below were counted by earlier tiles
    const int key0 = XATTN_KEY0(t);   // first key the tile holds
    const bool masked = key0 < lo || key0 + KT > L;
    const float mc = masked
        ? softmax_max<D, KSPLIT, true>(s_cur, st, kh, key0, lo, L, c, thr, lane)
        : softmax_max<D, KSPLIT, false>(s_cur, st, kh, key0, lo, L, c, thr, lane);
    softmax_exp<D, KSPLIT>(s_cur, pf, st, c, mc);
    pv_tile<D, KSPLIT>(tiles + (NSTAGE + t % NSTAGE) * Gm::TILE_BYTES, pf, st, kh, fo);
  }
#undef XATTN_KEY0

  // ---- Unshared stage from the gathered token blocks, on the matrix
  // cores: key half kh takes blocks kh, kh + KSPLIT, ... of its row group;
  // block 0 and the chunks copied in the loop (chunk c in stage
  // (chunk_t0 + c + 3) % NSTAGE) first, then any other chunks one at a time
  // through stage 0.
  {
    if (lds_tokens) {
      const int n_pref = min(n_chunks, max(0, n_tiles - 1 - chunk_t0));
      const int grow = row0 + rg * 32;
      const int gfirst = grow / G;
      const int n_valid = max(0, min((grow + 31) / G, BW - 1) - gfirst + 1) * nlev;
      // this row's tokens: its beam's nlev levels, within the group's valid tokens
      const int tok_lo = ((grow + ql) / G - gfirst) * nlev;
      const int tok_hi = min(tok_lo + nlev, n_valid);
      wait_vm_lgkm0<0>();
      lds_barrier();  // the blocks are in; every wave is done with the prompt tiles
      // ch = -1: block 0 in its region; ch >= 0: chunk ch
#pragma unroll 1
      for (int ch = -1; ch < n_chunks; ++ch) {
        const uint8_t *kt, *vt;
        if (ch < 0) {
          kt = XATTN_SK;
          vt = XATTN_SV;
        } else if (ch < n_pref) {
          const int sg = (chunk_t0 + ch + 3) % NSTAGE;
          kt = tiles + sg * Gm::TILE_BYTES;
          vt = tiles + (NSTAGE + sg) * Gm::TILE_BYTES;
        } else {
          lds_barrier();  // no wave still reads stage 0
          token_chunk_copy<D, WAVES>(XATTN_KT(0), XATTN_VT(0), cplan, ukg, uvg, tmap, ch, wave);
          wait_vm_lgkm0<0>();
          lds_barrier();
          kt = XATTN_KT(0);
          vt = XATTN_VT(0);
        }
#pragma unroll 1
        for (int b = kh; b < n_blk; b += KSPLIT) {
          const int gb = b * RG + rg;
          if ((gb == 0) != (ch < 0) || (gb > 0 && ((gb - 1) >> 1) != ch)) continue;
          const int off = gb == 0 ? 0 : 32 * ((gb - 1) & 1) * Gm::RB;
          if constexpr (TAPS)
            token_block<D, KSPLIT>(su, qf, kt + off, vt + off, fo, kh, 32 * b, tok_lo, tok_hi, c,
                                   thr, lane);
          else
            token_block<D, KSPLIT>(st, qf, kt + off, vt + off, fo, kh, 32 * b, tok_lo, tok_hi, c,
                                   thr, lane);
        }
      }
    }
  }
#undef XATTN_SK
#undef XATTN_SV

  // ---- the second key half hands its state to the first through LDS
  // (stage buffer rg holds row group rg's exchange)
  if constexpr (KSPLIT == 2) {
    static_assert(RG <= NSTAGE, "one stage buffer per row group");
    static_assert(NDB * 16 * 64 * 4 <= Gm::TILE_BYTES, "the exchanged O must fit a K tile");
    wait_vm_lgkm0<0>();
    lds_barrier();  // every wave is done with the tile stages
    if (p.anc_out && walk_here && k == 0 && split == 0) {
      // the ancestor slots this workgroup walked, for the beams whose first
      // query row lies in its block: anc_out [R][step + 1][BW]
      const int bf = (row0 + G - 1) / G;
      const int n = (min(row0 + ROWS, p.M) + G - 1) / G - bf;
      for (int i = tid; i < n * (step + 1); i += NT) {
        const int bi = i / (step + 1), t = i - bi * (step + 1);
        p.anc_out[((int64_t)r * (step + 1) + t) * BW + bf + bi] = anc_lds[(bf - b_lo + bi) * (step + 1) + t];
      }
    }
    float4 *xo = reinterpret_cast<float4 *>(XATTN_KT(rg));
    float *xs = reinterpret_cast<float *>(XATTN_VT(rg));
    if (kh == 1) half_put<D>(st, xo, xs, lane);
    __syncthreads();
    if constexpr (TAPS) {
      // the Shared states, then the Unshared states, through the same buffers
      if (kh == 0) half_merge<D>(st, xo, xs, c, lane);
      __syncthreads();
      if (kh == 1) half_put<D>(su, xo, xs, lane);
      __syncthreads();
      if (kh == 1) return;
      half_merge<D>(su, xo, xs, c, lane);
    } else {
      // the normalised rows of the plain path go out through LDS, stored by
      // both key halves (below); the key-split path leaves the writing to
      // key half 0
      if (kh == 1 && p.n_split > 1) return;
      if (kh == 0) half_merge<D>(st, xo, xs, c, lane);
    }
  }

  // ---- Merge / epilogue
  const int64_t n_rows_all = (int64_t)p.R * BW * p.Hq;
  const int64_t ri = qoff / D;
  if constexpr (!TAPS) {
    if (p.n_split > 1) {
      // one key split's partial (m, l, unnormalised O); merge_splits_kernel
      // combines the splits and writes out
      if (!valid) return;
      const int64_t pr = split * n_rows_all + ri;
      const float lt = pair_sum(st.l);
      if (hl == 0) {
        p.part_ml[pr * 2 + 0] = st.m;
        p.part_ml[pr * 2 + 1] = lt;
      }
      float *po = p.part_o + pr * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4 *>(po + db * 32 + 8 * j + 4 * hl) =
              make_float4(st.O[db][4 * j], st.O[db][4 * j + 1], st.O[db][4 * j + 2],
                          st.O[db][4 * j + 3]);
      return;
    }
  }
  if constexpr (TAPS) {
    // the Shared partial (m, l, O) and the Unshared partial, each on its
    // own, then their explicit OnlineSoftmax merge
    const float ls = pair_sum(st.l), lu = pair_sum(su.l);
    const float ms = st.m, mu = su.m;
    const float inv_s = ls > 0.f ? 1.f / ls : 0.f;
    const float inv_u = 1.f / lu;
    const float mm = fmaxf(ms, mu);
    const float ws = ls > 0.f ? ls * __builtin_amdgcn_exp2f((ms - mm) * c) : 0.f;
    const float wu = lu * __builtin_amdgcn_exp2f((mu - mm) * c);
    const float inv_z = 1.f / (ws + wu);
    if (valid) {
      if (p.stage_ml && hl == 0) {
        p.stage_ml[ri * 2 + 0] = ls > 0.f ? ms * p.scale : -INFINITY;
        p.stage_ml[ri * 2 + 1] = ls;
        p.stage_ml[(n_rows_all + ri) * 2 + 0] = mu * p.scale;
        p.stage_ml[(n_rows_all + ri) * 2 + 1] = lu;
      }
      if (p.stage_o) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int d = db * 32 + 8 * (e / 4) + 4 * hl + e % 4;
            p.stage_o[ri * D + d] = st.O[db][e] * inv_s;
            p.stage_o[(n_rows_all + ri) * D + d] = su.O[db][e] * inv_u;
          }
      }
      if (p.lse && hl == 0) p.lse[ri] = mm * p.scale + __logf(ws + wu);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      st.O[db] = (st.O[db] * (inv_s * ws) + su.O[db] * (inv_u * wu)) * inv_z;
  } else {
    if constexpr (KSPLIT == 2) {
      // Row group rg's 32 normalised rows as bf16 in LDS (V tile of stage
      // rg, past the exchanged m and l; row-major, 16-byte slots permuted by
      // swz), then stored by both waves of the group as whole rows, 16
      // bytes per lane: 64 / SLOTS rows per store instruction, where the
      // accumulator layout would give 8 bytes of each of 32 rows.
      static_assert(4096 + 32 * Gm::RB <= Gm::TILE_BYTES, "the staged rows must fit a V tile");
      uint8_t *ost = tiles + (NSTAGE + rg) * Gm::TILE_BYTES + 4096;
      if (kh == 0) {
        const float lt = pair_sum(st.l);
        const float inv = 1.f / lt;
        if (valid && p.lse && hl == 0) p.lse[ri] = st.m * p.scale + __logf(lt);
        const int osw = Gm::swz(ql);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x4 pk = {(__bf16)(st.O[db][4 * j + 0] * inv),
                               (__bf16)(st.O[db][4 * j + 1] * inv),
                               (__bf16)(st.O[db][4 * j + 2] * inv),
                               (__bf16)(st.O[db][4 * j + 3] * inv)};
            *reinterpret_cast<bf16x4 *>(ost + ql * Gm::RB + (((4 * db + j) ^ osw) << 4) +
                                        hl * 8) = pk;
          }
      }
      __syncthreads();
      constexpr int NCH = 32 * Gm::SLOTS / (KSPLIT * 64);   // store instructions per wave
#pragma unroll
      for (int n = 0; n < NCH; ++n) {
        const int idx = (n * KSPLIT + kh) * 64 + lane;
        const int orow = idx / Gm::SLOTS, ch = idx % Gm::SLOTS;
        const uint4 v =
            *reinterpret_cast<const uint4 *>(ost + orow * Gm::RB + ((ch ^ Gm::swz(orow)) << 4));
        const int grr = row0 + rg * 32 + orow;
        if (grr < p.M) {
          const int gb = grr / G;
          const int64_t go = (((int64_t)r * BW + gb) * p.Hq + k * G + (grr - gb * G)) * D;
          // written once: past the caches (non-temporal)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                      reinterpret_cast<u32x4 *>(og + go + ch * 8));
        }
      }
      return;
    } else {
      const float lt = pair_sum(st.l);
      const float inv = 1.f / lt;
      if (valid && p.lse && hl == 0) p.lse[ri] = st.m * p.scale + __logf(lt);
#pragma unroll
      for (int db = 0; db < NDB; ++db) st.O[db] *= inv;
    }
  }
#undef XATTN_KT
#undef XATTN_VT
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

// ---------------------------------------------------------------------------
// The paired variant, for grids of at least two workgroups per compute unit.
// One wave per row group of 32 query rows takes whole tiles of KT2 = 32
// keys (no key halves, so no exchange of halves at the end), the tile ring
// has NSTAGE2 = 4 stages, and the q rows and generated-token blocks pass
// through ring stages, so a workgroup needs at most 80 KiB of LDS and two
// of them share a compute unit.  The two waves on a SIMD then belong to
// different workgroups: neither waits at the other's barrier, one's
// softmax runs while the other's matrix products do, and one workgroup's
// prologue and epilogue run under the other's tile loop.  The per-tile work
// of a wave is the same as in decode_bf16_kernel (one 32-key block against
// its 32 rows), done by the same helpers.
constexpr int KT2 = 32;       // keys per tile
constexpr int NSTAGE2 = 4;    // ring depth (tiles in flight = NSTAGE2 - 1)

template <int D>
constexpr int kPairedLdsBytes = 2 * NSTAGE2 * TileGeom<D, KT2>::TILE_BYTES;

// One wave copies a whole generated-token block (32 rows of K to kt, of V
// to vt, in the tile layout): block gb of the row block (TokenMap).
template <int D, int RG>
__device__ __forceinline__ void token_block_copy_wave(uint8_t *kt, uint8_t *vt,
                                                      const uint16_t *ukg, const uint16_t *uvg,
                                                      const TokenMap<RG> &tm, int gb, int lane) {
  using Gm = TileGeom<D>;
  constexpr int NQ = 32 * Gm::RB / 1024;  // 1 KiB copies per K (or V) block
#pragma unroll
  for (int qi = 0; qi < 2 * NQ; ++qi) {
    const bool is_v = qi >= NQ;
    const int q = is_v ? qi - NQ : qi;
    const int row = q * Gm::ROWS_PER_COPY + lane / Gm::SLOTS;
    const int64_t e = tm.row_elem(gb, row, D);
    const uint8_t *src = reinterpret_cast<const uint8_t *>((is_v ? uvg : ukg) + e) +
                         (((lane % Gm::SLOTS) ^ Gm::swz(row)) << 4);
    dma16(src, (is_v ? vt : kt) + q * 1024);
  }
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

template <int D, int RG, bool TAPS>
__global__ __launch_bounds__(RG * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_bf16_paired_kernel(DecodeParams p) {
  constexpr int WAVES = RG;
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = RG * 32;
  constexpr int NKS = D / 16;           // k-steps of the QK contraction
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int KS = 2;                 // the helpers' unit: one 32-key block per wave
  using Gm = TileGeom<D, KT2>;
  constexpr int VREG = kVRegionOffset<D, KT2, NSTAGE2>();
  constexpr int CPW = Gm::COPIES / WAVES;   // wave-wide copies per wave per tile
  static_assert(RG <= NSTAGE2, "one ring stage per row group for its token blocks");
  static_assert(32 * Gm::RB == Gm::TILE_BYTES && Gm::TILE_BYTES == NKS * 1024,
                "a row group's 32 q rows (or token rows) fill one tile of NKS 1 KiB copies");

  // K tiles of stages 0..3, then V tiles of stages 0..3
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[kPairedLdsBytes<D>];
  // dynamic: ancestor slots [beams of the block][step + 1], then (when
  // staged) the parent rows [step][BW] of levels 1..step
  extern __shared__ int32_t dyn_lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int rg = __builtin_amdgcn_readfirstlane(tid >> 6);  // row group = wave
  const int hl = lane >> 5;
  const int ql = lane & 31;

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rb = lb % p.n_rb;
  const int split = (lb / p.n_rb) % p.n_split;
  const int unit = lb / p.n_rb / p.n_split;
  const int r = __builtin_amdgcn_readfirstlane(unit / p.Hkv);
  const int k = unit % p.Hkv;
  const int G = p.G, BW = p.BW, step = p.step;
  const int L = clampi(p.prompt_len[r], 0, p.Lmax);
  const float c = p.scale_log2;
  const float thr = p.lazy_log2 / c;

  const int row0 = rb * ROWS;
  const int b_lo = row0 / G;
  const int nb = (min(row0 + ROWS, p.M) - 1) / G - b_lo + 1;
  int32_t *anc_lds = dyn_lds;
  int32_t *par_lds = dyn_lds + nb * (step + 1);
  const bool walk_here = p.anc == nullptr;
  const bool staged = walk_here && p.stage_par != 0;

#define XP_KT(S) (tiles + (S) * Gm::TILE_BYTES)
#define XP_VT(S) (tiles + (NSTAGE2 + (S)) * Gm::TILE_BYTES)

  // ---- copies that depend on nothing: the parent rows for the walk, and
  // this wave's q rows, laid out like a tile (row-major, 16-byte slots
  // permuted by swz) in ring stage 2 + rg / 2 (K buffer for even rg, V for
  // odd); tiles 2 and 3 go there only after every wave holds its q.
  const int32_t *par = p.parent_idx + (int64_t)r * p.S * BW;
  if (staged) {
    const int n_par = step * BW;
    for (int c0 = rg * 64; c0 < n_par; c0 += WAVES * 64)
      dma4(par + BW + min(c0 + lane, n_par - 1), par_lds + c0);
  }
  const uint16_t *qg = static_cast<const uint16_t *>(p.q);
  uint16_t *og = static_cast<uint16_t *>(p.out);
  const int row = row0 + rg * 32 + ql;
  const bool valid = row < p.M;
  const int rr = valid ? row : p.M - 1;
  const int beam = rr / G;
  const int64_t qoff = (((int64_t)r * BW + beam) * p.Hq + k * G + rr % G) * D;
  uint8_t *qlds = (rg & 1) ? XP_VT(2 + rg / 2) : XP_KT(2 + rg / 2);
#pragma unroll
  for (int n = 0; n < NKS; ++n) {
    const int qr = n * Gm::ROWS_PER_COPY + lane / Gm::SLOTS;   // row of the group
    const int qrr = min(row0 + rg * 32 + qr, p.M - 1);
    const int qb = qrr / G;
    const int64_t qro = (((int64_t)r * BW + qb) * p.Hq + k * G + (qrr - qb * G)) * D;
    dma16<false>(qg + qro + (((lane % Gm::SLOTS) ^ Gm::swz(qr)) << 3), qlds + n * 1024);
  }

  const uint16_t *ukg = static_cast<const uint16_t *>(p.unshared_k) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  const uint16_t *uvg = static_cast<const uint16_t *>(p.unshared_v) +
                        ((int64_t)r * p.Hkv + k) * p.S * BW * D;
  const uint16_t *skg = static_cast<const uint16_t *>(p.shared_k) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  const uint16_t *svg = static_cast<const uint16_t *>(p.shared_v) +
                        ((int64_t)r * p.Hkv + k) * p.Lmax * D;
  CopyPlan<D, WAVES, KT2> cplan;
  cplan.init(rg, lane);
  // tiles 0 and 1 (keys [0, 2 KT2)) before the prompt length is known: they
  // are right whenever the prompt has more than two tiles
  const bool speculate = p.n_split == 1 && p.Lmax >= 2 * KT2;
  if (speculate) {
    tile_copy<D, WAVES, false, false, KT2>(XP_KT(0), XP_VT(0), cplan, skg, svg, 0, 0, rg);
    tile_copy<D, WAVES, false, false, KT2>(XP_KT(1), XP_VT(1), cplan, skg, svg, KT2, 0, rg);
  }
  // the prompt's tiles split evenly over the key splits: this workgroup
  // takes tiles [t_base, t_base + n_tiles); the last window of the prompt
  // is shifted back to end at L (its keys already counted get masked)
  const int n_tiles_all = (L + KT2 - 1) / KT2;
  const int t_base = split * n_tiles_all / p.n_split;
  const int n_tiles = (split + 1) * n_tiles_all / p.n_split - t_base;
  const int last_key0 = L >= KT2 ? L - KT2 : 0;
#define XP_KEY0(T) (t_base + (T) + 1 < n_tiles_all ? (t_base + (T)) * KT2 : last_key0)
  const bool spec_ok = speculate && n_tiles > 2;

  // ---- the parent rows and q are in (older than the speculative tiles);
  // walk the ancestor chains of the block's beams, take q into registers
  if (speculate)
    wait_vm_lgkm0<TAPS ? 0 : (2 * CPW)>();
  else
    wait_vm_lgkm0<0>();
  lds_barrier();   // every wave's parent and q copies have landed
  if (walk_here) {
    for (int i = tid; i < nb; i += NT) {
      int a = b_lo + i;
      int32_t *dst = anc_lds + i * (step + 1);
      dst[step] = a;
      for (int t = step; t >= 1; --t) {
        a = clampi(staged ? par_lds[(t - 1) * BW + a] : par[(int64_t)t * BW + a], 0, BW - 1);
        dst[t - 1] = a;
      }
    }
  }
  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8 *>(qlds + ql * Gm::RB +
                                                (((2 * ks + hl) ^ Gm::swz(ql)) << 4));
  wait_lgkm0();
  lds_barrier();   // the ancestor slots are visible; every wave holds its q
  if (!spec_ok) {
    if (speculate) wait_vm_lgkm0<0>();   // before stages 0 and 1 are written again
    if (n_tiles > 0) {
      if (L < KT2)
        tile_copy<D, WAVES, true, false, KT2>(XP_KT(0), XP_VT(0), cplan, skg, svg, 0, L, rg);
      else
        tile_copy<D, WAVES, false, false, KT2>(XP_KT(0), XP_VT(0), cplan, skg, svg, XP_KEY0(0),
                                               L, rg);
    }
    if (n_tiles > 1)
      tile_copy<D, WAVES, false, false, KT2>(XP_KT(1), XP_VT(1), cplan, skg, svg, XP_KEY0(1), L,
                                             rg);
  }
  if (n_tiles > 2)
    tile_copy<D, WAVES, false, false, KT2>(XP_KT(2), XP_VT(2), cplan, skg, svg, XP_KEY0(2), L, rg);

  // st: the online-softmax state of the row; with TAPS, of the Shared stage
  // alone, and su that of the Unshared stage
  Rows<D> st, su;
  st.clear();
  su.clear();
  if (!walk_here) {
    // deep chains: the Unshared stage was computed beforehand, one workgroup
    // per (request, beam, KV head); key split 0 starts from its partial
    if (split == 0) {
      if constexpr (TAPS)
        seed_rows<D>(su, p, qoff / D, hl);
      else
        seed_rows<D>(st, p, qoff / D, hl);
    }
    // complete these compiler-counted loads before the tile loop (see the
    // same step in decode_bf16_kernel)
    wait_vm_lgkm0<0>();
  }

  // ---- tile 0 is in once all but the copies younger than it are
  if (n_tiles > 2)
    wait_vm_lgkm0<TAPS ? 0 : (2 * CPW)>();
  else if (n_tiles > 1)
    wait_vm_lgkm0<TAPS ? 0 : CPW>();
  else
    wait_vm_lgkm0<0>();
  lds_barrier();   // tile 0 is visible

  // ---- Shared stage.  Per tile t (in stage t % 4) but the last: wait for
  // tile t + 1 and synchronise, finish the row maxima of tile t, issue the
  // S^T MFMAs of tile t + 1 interleaved with the exponentials of tile t,
  // then tile t's PV MFMAs (with tile t + 1's row maxima between them),
  // then copy tile t + 3 into the stage tile t - 1 used.
  FragOffsets<D, VREG> fo;
  fo.init(0, 1, lane);
  f32x16 s_cur[1], s_next[1];
  bf16x8 pf[2];
  if (n_tiles > 0) qk_tile<D, KS, VREG>(XP_KT(0), qf, s_cur, fo);
  float tmax_cur = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) tmax_cur = fmaxf(tmax_cur, s_cur[0][e]);
#define XP_TILE_STEP(ST)                                                              \
  {                                                                                   \
    const int t = t0 + (ST);                                                          \
    if (t + 1 >= n_tiles) break;                                                      \
    /* tile t + 1 is in once all but the copy younger than it (tile t + 2, */         \
    /* copied at step t - 1 or, for t = 0, in the prologue) are */                   \
    if (t + 2 < n_tiles)                                                              \
      wait_vm_lgkm0<TAPS ? 0 : CPW>();                                                \
    else                                                                              \
      wait_vm_lgkm0<0>();                                                             \
    lds_barrier();                                                                    \
    const float mc = softmax_max_finish<D>(tmax_cur, st, c, thr);                     \
    qk_next_with_exp<D, KS, VREG>(XP_KT(((ST) + 1) % NSTAGE2), qf, s_next, s_cur, pf, st, \
                                  c, mc, fo);                                         \
    pv_tile_max<D, KS, VREG>(XP_VT(ST), pf, st, 0, fo, s_next, tmax_cur);             \
    if (t + 3 < n_tiles)                                                              \
      tile_copy<D, WAVES, false, true, KT2>(XP_KT(((ST) + 3) % NSTAGE2),              \
                                            XP_VT(((ST) + 3) % NSTAGE2), cplan, skg, svg, \
                                            XP_KEY0(t + 3), L, rg);                   \
    s_cur[0] = s_next[0];                                                             \
  }
  static_assert(NSTAGE2 == 4, "the tile loop below is unrolled for 4 stages");
  for (int t0 = 0; t0 + 1 < n_tiles; t0 += NSTAGE2) {
    XP_TILE_STEP(0)
    XP_TILE_STEP(1)
    XP_TILE_STEP(2)
    XP_TILE_STEP(3)
  }
#undef XP_TILE_STEP
  if (n_tiles > 0) {  // the last tile: every copy has landed
    const int t = n_tiles - 1;
    const int lo = (t_base + t) * KT2;   // keys below were counted by earlier tiles
    const int key0 = XP_KEY0(t);         // first key the tile holds
    const bool masked = key0 < lo || key0 + KT2 > L;
    const float mc = masked ? softmax_max<D, KS, true>(s_cur, st, 0, key0, lo, L, c, thr, lane)
                            : softmax_max<D, KS, false>(s_cur, st, 0, key0, lo, L, c, thr, lane);
    softmax_exp<D, KS>(s_cur, pf, st, c, mc);
    pv_tile<D, KS, VREG>(XP_VT(t % NSTAGE2), pf, st, 0, fo);
  }
#undef XP_KEY0

  wait_vm_lgkm0<0>();
  lds_barrier();   // every wave is done with the ring
  if (p.anc_out && walk_here && k == 0 && split == 0) {
    // the ancestor slots this workgroup walked, for the beams whose first
    // query row lies in its block: anc_out [R][step + 1][BW]
    const int bf = (row0 + G - 1) / G;
    const int n = (min(row0 + ROWS, p.M) + G - 1) / G - bf;
    for (int i = tid; i < n * (step + 1); i += NT) {
      const int bi = i / (step + 1), t = i - bi * (step + 1);
      p.anc_out[((int64_t)r * (step + 1) + t) * BW + bf + bi] =
          anc_lds[(bf - b_lo + bi) * (step + 1) + t];
    }
  }

  // ---- Unshared stage from the generated-token rows, on the matrix cores:
  // row group rg's tokens (its beams' levels, TokenMap) in blocks of 32
  // rows, each gathered by the wave into its own ring stage and contracted
  // like a 32-key tile under a block-diagonal mask, into the same state
  // (with TAPS, into su)
  if (walk_here) {
    const int nlev = step + 1;
    const int nbr_max = (32 % G == 0) ? 32 / G : 32 / G + 2;  // beams 32 rows can touch
    const int n_blk = (nbr_max * nlev + 31) / 32;
    TokenMap<RG> tmap;
    tmap.init(anc_lds, n_blk, nlev, BW, nb, G, row0, b_lo);
    const int grow = row0 + rg * 32;
    const int gfirst = grow / G;
    const int n_valid = max(0, min((grow + 31) / G, BW - 1) - gfirst + 1) * nlev;
    const int tok_lo = ((grow + ql) / G - gfirst) * nlev;
    const int tok_hi = min(tok_lo + nlev, n_valid);
#pragma unroll 1
    for (int b = 0; b < n_blk; ++b) {
      token_block_copy_wave<D, RG>(XP_KT(rg), XP_VT(rg), ukg, uvg, tmap, b * RG + rg, lane);
      wait_vm_lgkm0<0>();   // this wave's own copies: no other wave uses stage rg now
      if constexpr (TAPS)
        token_block<D, KS, VREG>(su, qf, XP_KT(rg), XP_VT(rg), fo, 0, 32 * b, tok_lo, tok_hi, c,
                                 thr, lane);
      else
        token_block<D, KS, VREG>(st, qf, XP_KT(rg), XP_VT(rg), fo, 0, 32 * b, tok_lo, tok_hi, c,
                                 thr, lane);
    }
  }

  // ---- Merge / epilogue
  const int64_t n_rows_all = (int64_t)p.R * BW * p.Hq;
  const int64_t ri = qoff / D;
  if constexpr (!TAPS) {
    if (p.n_split > 1) {
      // one key split's partial (m, l, unnormalised O); merge_splits_kernel
      // combines the splits and writes out
      if (!valid) return;
      const int64_t pr = split * n_rows_all + ri;
      const float lt = pair_sum(st.l);
      if (hl == 0) {
        p.part_ml[pr * 2 + 0] = st.m;
        p.part_ml[pr * 2 + 1] = lt;
      }
      float *po = p.part_o + pr * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4 *>(po + db * 32 + 8 * j + 4 * hl) =
              make_float4(st.O[db][4 * j], st.O[db][4 * j + 1], st.O[db][4 * j + 2],
                          st.O[db][4 * j + 3]);
      return;
    }
    // the row group's 32 normalised rows as bf16 in the wave's own K stage
    // (row-major, 16-byte slots permuted by swz), then stored whole, 16
    // bytes per lane
    const float lt = pair_sum(st.l);
    const float inv = 1.f / lt;
    if (valid && p.lse && hl == 0) p.lse[ri] = st.m * p.scale + __logf(lt);
    uint8_t *ost = XP_KT(rg);
    const int osw = Gm::swz(ql);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 pk = {(__bf16)(st.O[db][4 * j + 0] * inv), (__bf16)(st.O[db][4 * j + 1] * inv),
                           (__bf16)(st.O[db][4 * j + 2] * inv), (__bf16)(st.O[db][4 * j + 3] * inv)};
        *reinterpret_cast<bf16x4 *>(ost + ql * Gm::RB + (((4 * db + j) ^ osw) << 4) + hl * 8) = pk;
      }
    wait_lgkm0();
    constexpr int NCH = 32 * Gm::SLOTS / 64;   // store instructions per wave
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int idx = n * 64 + lane;
      const int orow = idx / Gm::SLOTS, ch = idx % Gm::SLOTS;
      const uint4 v =
          *reinterpret_cast<const uint4 *>(ost + orow * Gm::RB + ((ch ^ Gm::swz(orow)) << 4));
      const int grr = row0 + rg * 32 + orow;
      if (grr < p.M) {
        const int gb = grr / G;
        const int64_t go = (((int64_t)r * BW + gb) * p.Hq + k * G + (grr - gb * G)) * D;
        // written once: past the caches (non-temporal)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                    reinterpret_cast<u32x4 *>(og + go + ch * 8));
      }
    }
  } else {
    // the Shared partial (m, l, O) and the Unshared partial, each on its
    // own, then their explicit OnlineSoftmax merge
    const float ls = pair_sum(st.l), lu = pair_sum(su.l);
    const float ms = st.m, mu = su.m;
    const float inv_s = ls > 0.f ? 1.f / ls : 0.f;
    const float inv_u = 1.f / lu;
    const float mm = fmaxf(ms, mu);
    const float ws = ls > 0.f ? ls * __builtin_amdgcn_exp2f((ms - mm) * c) : 0.f;
    const float wu = lu * __builtin_amdgcn_exp2f((mu - mm) * c);
    const float inv_z = 1.f / (ws + wu);
    if (!valid) return;
    if (p.stage_ml && hl == 0) {
      p.stage_ml[ri * 2 + 0] = ls > 0.f ? ms * p.scale : -INFINITY;
      p.stage_ml[ri * 2 + 1] = ls;
      p.stage_ml[(n_rows_all + ri) * 2 + 0] = mu * p.scale;
      p.stage_ml[(n_rows_all + ri) * 2 + 1] = lu;
    }
    if (p.stage_o) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int d = db * 32 + 8 * (e / 4) + 4 * hl + e % 4;
          p.stage_o[ri * D + d] = st.O[db][e] * inv_s;
          p.stage_o[(n_rows_all + ri) * D + d] = su.O[db][e] * inv_u;
        }
    }
    if (p.lse && hl == 0) p.lse[ri] = mm * p.scale + __logf(ws + wu);
    uint16_t *op = og + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x16 o = (st.O[db] * (inv_s * ws) + su.O[db] * (inv_u * wu)) * inv_z;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 pk = {(__bf16)o[4 * j + 0], (__bf16)o[4 * j + 1], (__bf16)o[4 * j + 2],
                           (__bf16)o[4 * j + 3]};
        *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * j + 4 * hl) = pk;
      }
    }
  }
#undef XP_KT
#undef XP_VT
}

// Launch geometry of one variant: `threads` per workgroup of `rows` query
// rows, `static_lds` bytes of static LDS, and at most `budget` bytes of LDS
// per workgroup (the paired variant keeps two workgroups per CU).
Bf16Geometry geometry_for(const DecodeParams &p, int rows, int threads, int static_lds,
                          int budget, bool paired) {
  Bf16Geometry g{};
  g.rows = rows;
  g.threads = threads;
  g.paired = paired;
  g.grid = (int64_t)p.R * p.Hkv * ((p.M + rows - 1) / rows) * p.n_split;
  g.static_lds = static_lds;
  g.beams_per_block = beams_per_block(rows, p.G, p.BW);
  g.dyn_lds = 0;
  g.stage_par = false;
  if (p.anc == nullptr) {
    // ancestor slots [beams of the block][step + 1]
    g.dyn_lds = g.beams_per_block * (p.step + 1) * (int)sizeof(int32_t);
    // parent rows, copied 64 ints per wave instruction: whole rounds of 64
    const int par_bytes = (p.step * p.BW + 63) / 64 * 64 * (int)sizeof(int32_t);
    if (p.step > 0 && (int64_t)p.step * p.BW <= kParentLdsInts &&
        g.static_lds + g.dyn_lds + par_bytes <= budget) {
      g.stage_par = true;
      g.dyn_lds += par_bytes;
    }
  }
  return g;
}

// Rows per workgroup: 32 (1 row group) or 64 (2) for few query rows per
// (request, KV head); otherwise 128 rows in 4 row groups.
int rows_per_block(int M) { return M <= 32 ? 32 : (M <= 64 ? 64 : 128); }

// Workgroups of the paired variant that keep every compute unit's two
// slots busy (256 CUs).
constexpr int64_t kPairedMinGrid = 512;

template <int D>
Bf16Geometry geometry_d(const DecodeParams &p) {
  const int rows = rows_per_block(p.M);
  if (rows == 128) {
    const Bf16Geometry g = geometry_for(p, 128, 4 * 64, kPairedLdsBytes<D>, kLdsLimit / 2, true);
    if (g.grid >= kPairedMinGrid && g.static_lds + g.dyn_lds <= kLdsLimit / 2) return g;
  }
  return geometry_for(p, rows, rows / 32 * 2 * 64, kTilesLdsBytes<D>, kLdsLimit, false);
}

template <int D, int RG, bool TAPS>
hipError_t launch_cfg(const DecodeParams &p0, const Bf16Geometry &g, hipStream_t stream,
                      LaunchEvents ev) {
  DecodeParams p = p0;
  p.n_rb = (p.M + g.rows - 1) / g.rows;
  if (TAPS && p.n_split != 1) return hipErrorInvalidValue;
  if (g.grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (g.static_lds + g.dyn_lds > (g.paired ? kLdsLimit / 2 : kLdsLimit))
    return hipErrorInvalidConfiguration;
  p.stage_par = g.stage_par ? 1 : 0;
  const uint32_t dyn = (uint32_t)g.dyn_lds;
  auto kernel = decode_bf16_kernel<D, RG, 2, TAPS>;
  if constexpr (RG == 4) {
    if (g.paired) kernel = decode_bf16_paired_kernel<D, RG, TAPS>;
  } else if (g.paired) {
    return hipErrorInvalidConfiguration;   // the paired variant runs 128-row workgroups only
  }
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)g.grid), dim3(g.threads), dyn, stream, ev.start,
                          ev.stop, 0u, p);
  else
    hipLaunchKernelGGL(kernel, dim3((unsigned)g.grid), dim3(g.threads), dyn, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams &p, bool taps, hipStream_t stream, LaunchEvents ev) {
  const Bf16Geometry g = geometry_d<D>(p);
  if (taps) {
    if (g.rows == 32) return launch_cfg<D, 1, true>(p, g, stream, ev);
    if (g.rows == 64) return launch_cfg<D, 2, true>(p, g, stream, ev);
    return launch_cfg<D, 4, true>(p, g, stream, ev);
  }
  if (g.rows == 32) return launch_cfg<D, 1, false>(p, g, stream, ev);
  if (g.rows == 64) return launch_cfg<D, 2, false>(p, g, stream, ev);
  return launch_cfg<D, 4, false>(p, g, stream, ev);
}

// Merge of the key splits' partials (OnlineSoftmax over the splits, the
// combine of the xGR summary's Merge stage applied to n_split partials):
// one wave per query row, D / 64 dims per lane.  m = max_s m_s, weights
// w_s = exp2((m_s - m) * scale_log2), out = sum_s w_s o_s / sum_s w_s l_s.
template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeParams p) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t n_rows_all = (int64_t)p.R * p.BW * p.Hq;
  const int64_t ri = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (ri >= n_rows_all) return;
  const float c = p.scale_log2;
  // every split's (m, l) and o loads go out together
  float ms[kMaxKeySplits], ls[kMaxKeySplits], os[kMaxKeySplits][PER];
#pragma unroll
  for (int sp = 0; sp < kMaxKeySplits; ++sp) {
    const bool in = sp < p.n_split;
    const int64_t pr = (in ? sp : 0) * n_rows_all + ri;
    const float2 ml = *reinterpret_cast<const float2 *>(p.part_ml + pr * 2);
    ms[sp] = in ? ml.x : -INFINITY;
    ls[sp] = in ? ml.y : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) os[sp][k] = in ? p.part_o[pr * D + lane * PER + k] : 0.f;
  }
  float m = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxKeySplits; ++sp) m = fmaxf(m, ms[sp]);
  float l = 0.f, acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxKeySplits; ++sp) {
    const float w = ms[sp] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ms[sp] - m) * c);
    l += ls[sp] * w;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] += os[sp][k] * w;
  }
  const float inv = 1.f / l;
  uint16_t *op = static_cast<uint16_t *>(p.out) + ri * D + lane * PER;
  if constexpr (PER == 2) {
    // the lane's two values as one 4-byte store, written once (non-temporal)
    const bf16x2 v = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
    __builtin_nontemporal_store(__builtin_bit_cast(uint32_t, v), reinterpret_cast<uint32_t *>(op));
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const __bf16 v = (__bf16)(acc[k] * inv);
      op[k] = *reinterpret_cast<const uint16_t *>(&v);
    }
  }
  if (p.lse && lane == 0) p.lse[ri] = m * p.scale + __logf(l);
}

}  // namespace

int bf16_rows_per_block(const DecodeParams &p) { return rows_per_block(p.M); }

Bf16Geometry bf16_geometry(const DecodeParams &p) {
  return p.D == 64 ? geometry_d<64>(p) : geometry_d<128>(p);
}

hipError_t launch_merge_splits_bf16(const DecodeParams &p, hipStream_t stream, LaunchEvents ev) {
  const int64_t rows = (int64_t)p.R * p.BW * p.Hq;
  const int64_t grid = (rows + 3) / 4;
  if (grid > 0x7fffffff || p.n_split < 2 || p.n_split > kMaxKeySplits)
    return hipErrorInvalidConfiguration;
  auto kernel = p.D == 64 ? merge_splits_kernel<64> : merge_splits_kernel<128>;
  if (p.D != 64 && p.D != 128) return hipErrorInvalidValue;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0u, stream, ev.start, ev.stop,
                          0u, p);
  else
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeParams &p, bool taps, hipStream_t stream,
                              LaunchEvents ev) {
  if (p.D == 64) return launch_d<64>(p, taps, stream, ev);
  if (p.D == 128) return launch_d<128>(p, taps, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace xattn
