// Beam selection for one decode step: the BW best of a request's BW x V
// candidates (xGR summary, section 2.2 "xBeam"; pools of 128x128 and
// 512x512 from its section 1).
//
// Every beam b proposes V candidates sorted by log-probability; candidate
// (b, j) scores the float32 sum cum[b] + logp[b][j], and the order is score
// descending, then parent beam ascending, then token id ascending.  The page
// keeps a global min-heap of BW entries and stops scanning a beam once its
// next candidate cannot enter the heap.  A heap is a serial structure, so
// this kernel keeps the idea -- sorted rows let a threshold cut every row's
// scan short -- and replaces the heap by a threshold search that a whole
// workgroup runs in LDS:
//
//   1. Sample.  The first c0 candidates of every row (c0 = min(V, 16384 /
//      BW)) are scored into LDS as order-preserving uint32 keys.
//   2. Threshold.  T0 = the BW-th largest sampled key, by radix selection.
//      The sample is a subset of the pool, so the true threshold T (the
//      BW-th largest key of the pool) is >= T0.
//   3. Early-terminating scans.  Per row, the number of candidates above and
//      at T0 is a binary search in the sampled prefix; only rows whose whole
//      prefix is >= T0 read further, 64 candidates a step, and stop at the
//      first candidate below T0.  No candidate at position >= BW can score
//      above T (BW earlier ones in its row would all beat it), so these
//      scans never go past position max(c0, min(V, BW)).
//   4. If fewer than BW candidates are above T0, then T = T0.  Otherwise the
//      candidates above T0 (at most 7711 for BW <= 512) are gathered into
//      LDS and T is their BW-th largest key.
//   5. Ties.  Every candidate above T is selected; the remaining slots go to
//      candidates equal to T in beam order, and inside the one beam that
//      gets only part of its ties, to the smallest token ids (a radix
//      selection over that beam's tie run, which may extend to the end of
//      its row).
//   6. The BW winners are ordered by (score desc, beam asc, token asc) with a
//      bitonic network (register shuffles within a wave, LDS across waves)
//      and written out.
//
// One 1024-thread workgroup per request; every loop is bounded by the
// shape, and indexes are clamped before every LDS or global access.
#include <hip/hip_ext.h>

#include "xattn_internal.h"

namespace xattn {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kSampleCap = 16384;   // sampled keys held in LDS
constexpr int kListCap = 8192;      // candidates above the sample threshold
constexpr int kMaxBW = kMaxTopkBeams;

struct TopkArgs {
  const float *cum;      // [R][BW]
  const float *logp;     // [R][BW][V]
  const int32_t *tok;    // [R][BW][V]
  float *score;          // [R] rows of BW, stride out_stride
  int32_t *parent;
  int32_t *token;
  int64_t out_stride;
  int32_t BW, V, c0;
};

struct Smem {
  uint32_t s0[kSampleCap];   // sampled keys, row b at b * c0
  uint32_t lkey[kListCap];   // gathered candidates: key
  uint32_t lidx[kListCap];   //                      beam << 16 | position
  float cum[kMaxBW];
  int32_t gt[kMaxBW];        // per row: candidates above T (then T0)
  int32_t ge[kMaxBW];        // per row: candidates at or above T
  int32_t off[kMaxBW];       // per row: exclusive prefix (gather / output)
  int32_t rows[kMaxBW];      // list of rows needing a longer scan
  uint64_t sa[kMaxBW];       // sort items: (~key) << 32 | beam
  uint32_t st[kMaxBW];       //             token ^ 0x80000000
  uint32_t hist[256];
  int32_t red[2 * kWaves];
  int32_t ctl[16];
};

// float -> uint32 with the same order; -0 maps to +0 so the two compare equal
__device__ inline uint32_t score_key(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_score(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

__device__ inline uint32_t cand_key(float cum, float lp) { return score_key(__fadd_rn(cum, lp)); }

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum of v over the block; every thread gets it.
__device__ int block_sum(int v, Smem &sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) sm.red[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += sm.red[w];
  __syncthreads();
  return t;
}

// min and max of v over the block
__device__ void block_minmax(uint32_t lo, uint32_t hi, Smem &sm, uint32_t &olo, uint32_t &ohi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }
  if (lane == 0) {
    sm.red[wave] = (int)lo;
    sm.red[kWaves + wave] = (int)hi;
  }
  __syncthreads();
  olo = 0xffffffffu;
  ohi = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    olo = min(olo, (uint32_t)sm.red[w]);
    ohi = max(ohi, (uint32_t)sm.red[kWaves + w]);
  }
  __syncthreads();
}

// Exclusive prefix sum of v over threads 0..kMaxBW-1 (the other threads pass
// 0); returns this thread's prefix, *total the sum.
__device__ int block_scan(int v, Smem &sm, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sm.red[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int x = sm.red[w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// The k-th largest (1 <= k <= n) of keys get(0..n-1), all in [lo, hi], by
// most-significant-digit radix selection over the bits below the common
// prefix of lo and hi.  Every thread of the block calls it and gets the
// result; *n_above = keys strictly greater than it.
template <class Get>
__device__ uint32_t kth_largest(Get get, int n, int k, uint32_t lo, uint32_t hi, Smem &sm,
                                int *n_above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (lo == hi) {
    *n_above = 0;
    return lo;
  }
  int bit = 32 - __clz(lo ^ hi);   // bits [0, bit) differ somewhere
  uint32_t prefix = hi & ~((bit == 32) ? 0xffffffffu : ((1u << bit) - 1u));
  uint32_t mask = ~((bit == 32) ? 0xffffffffu : ((1u << bit) - 1u));
  int krem = k;
  while (bit > 0) {
    const int w = bit < 8 ? bit : 8;
    const int shift = bit - w;
    const uint32_t dmask = (1u << w) - 1u;
    for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = get(i);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // bins 4*lane .. 4*lane+3; suffix sums over lanes from the top
      uint32_t h[4];
      uint32_t s = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = sm.hist[4 * lane + e];
        s += h[e];
      }
      uint32_t inc = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_down((int)inc, o);
        if (lane + o < 64) inc += t;
      }
      uint32_t above = inc - s;   // keys in bins of higher lanes
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (above < (uint32_t)krem && above + h[e] >= (uint32_t)krem) {
          sm.ctl[0] = 4 * lane + e;
          sm.ctl[1] = krem - (int)above;
        }
        above += h[e];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sm.ctl[0];
    krem = sm.ctl[1];
    __syncthreads();
    prefix |= d << shift;
    mask |= dmask << shift;
    bit = shift;
  }
  *n_above = k - krem;
  return prefix;
}

// Per-row counts above / at-or-above x over positions [from, to) of a sorted
// row, read from global memory 64 at a time, stopping at the first
// candidate below x; `equal_only` counts the run of candidates equal to x.
__device__ void scan_row(const float *lp, float cum, int from, int to, uint32_t x, int *n_gt,
                         int *n_ge) {
  const int lane = threadIdx.x & 63;
  int gt = 0, ge = 0;
  for (int j0 = from; j0 < to; j0 += 64) {
    const int j = j0 + lane;
    const bool in = j < to;
    const uint32_t key = in ? cand_key(cum, lp[j]) : 0u;
    const uint64_t bgt = __ballot(in && key > x);
    const uint64_t bge = __ballot(in && key >= x);
    gt += __popcll(bgt);
    ge += __popcll(bge);
    const int valid = min(64, to - j0);
    const uint64_t full = valid == 64 ? ~0ull : ((1ull << valid) - 1ull);
    if (bge != full) break;
  }
  *n_gt = gt;
  *n_ge = ge;
}

__global__ __launch_bounds__(kThreads) void beam_topk_kernel(TopkArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int BW = a.BW, V = a.V, c0 = a.c0;
  const int P = min(V, BW);        // no candidate at position >= P is above T
  const int Pc = max(c0, P);       // prefix every row's counts cover
  const float *cum = a.cum + (int64_t)r * BW;
  const float *logp = a.logp + (int64_t)r * BW * V;
  const int32_t *tok = a.tok + (int64_t)r * BW * V;

  for (int b = tid; b < BW; b += kThreads) {
    sm.cum[b] = cum[b];
    sm.sa[b] = ~0ull;   // every slot is written below when the rows are sorted
    sm.st[b] = ~0u;
  }
  __syncthreads();

  // 1. sample: the first c0 candidates of every row
  const int n0 = BW * c0;
  uint32_t lo = 0xffffffffu, hi = 0u;
  {
    int b = tid / c0, j = tid % c0;
    const int db = kThreads / c0, dj = kThreads % c0;
    for (int i = tid; i < n0; i += kThreads) {
      const uint32_t key = cand_key(sm.cum[b], logp[(int64_t)b * V + j]);
      sm.s0[i] = key;
      lo = min(lo, key);
      hi = max(hi, key);
      b += db;
      j += dj;
      if (j >= c0) {
        j -= c0;
        ++b;
      }
    }
  }
  block_minmax(lo, hi, sm, lo, hi);   // includes the barrier after the stores

  // 2. T0: the BW-th largest sampled key
  int above0;
  const uint32_t T0 = kth_largest([&](int i) { return sm.s0[i]; }, n0, BW, lo, hi, sm, &above0);

  // 3. per-row counts against T0 over the sampled prefix (binary search on
  //    the non-increasing keys); rows whose prefix is all >= T0 scan further
  if (tid == 0) sm.ctl[2] = 0;
  __syncthreads();
  for (int b = tid; b < BW; b += kThreads) {
    const uint32_t *row = sm.s0 + b * c0;
    int l = 0, h = c0;
    while (l < h) {
      const int m = (l + h) >> 1;
      if (row[m] > T0) l = m + 1; else h = m;
    }
    const int gt = l;
    h = c0;
    while (l < h) {
      const int m = (l + h) >> 1;
      if (row[m] >= T0) l = m + 1; else h = m;
    }
    sm.gt[b] = gt;
    sm.ge[b] = l;
    if (l == c0 && c0 < Pc) sm.rows[atomicAdd(&sm.ctl[2], 1)] = b;
  }
  __syncthreads();
  {
    const int n_ext = min(sm.ctl[2], BW);
    for (int e = wave; e < n_ext; e += kWaves) {
      const int b = sm.rows[e];
      int gt, ge;
      scan_row(logp + (int64_t)b * V, sm.cum[b], c0, Pc, T0, &gt, &ge);
      if (lane == 0) {
        sm.gt[b] += gt;
        sm.ge[b] += ge;
      }
    }
  }
  __syncthreads();
  int n_gt = block_sum(tid < BW ? sm.gt[tid] : 0, sm);

  // 4. the exact threshold
  uint32_t T = T0;
  if (n_gt >= BW) {
    // gather every candidate above T0 (positions < Pc) into the list
    int n_list;
    const int my = block_scan(tid < BW ? sm.gt[tid] : 0, sm, &n_list);
    if (tid < BW) sm.off[tid] = my;
    __syncthreads();
    n_list = min(n_list, kListCap);
    uint32_t llo = 0xffffffffu, lhi = 0u;
    for (int b = wave; b < BW; b += kWaves) {
      const int cnt = sm.gt[b], base = sm.off[b];
      for (int j = lane; j < cnt; j += 64) {
        const uint32_t key = j < c0 ? sm.s0[b * c0 + j]
                                    : cand_key(sm.cum[b], logp[(int64_t)b * V + j]);
        const int at = base + j;
        if (at < kListCap) {
          sm.lkey[at] = key;
          sm.lidx[at] = ((uint32_t)b << 16) | (uint32_t)j;
          llo = min(llo, key);
          lhi = max(lhi, key);
        }
      }
    }
    block_minmax(llo, lhi, sm, llo, lhi);
    int above;
    T = kth_largest([&](int i) { return sm.lkey[i]; }, n_list, BW, llo, lhi, sm, &above);
    // counts against T: every candidate >= T at positions < Pc is listed
    for (int b = tid; b < BW; b += kThreads) {
      sm.gt[b] = 0;
      sm.ge[b] = 0;
    }
    __syncthreads();
    for (int i = tid; i < n_list; i += kThreads) {
      const uint32_t key = sm.lkey[i];
      const int b = (int)(sm.lidx[i] >> 16);
      if (key > T) atomicAdd(&sm.gt[b], 1);
      if (key >= T) atomicAdd(&sm.ge[b], 1);
    }
    __syncthreads();
    n_gt = block_sum(tid < BW ? sm.gt[tid] : 0, sm);
  }

  // 5. ties: a run equal to T that reaches Pc may continue to the row's end
  if (tid == 0) sm.ctl[2] = 0;
  __syncthreads();
  for (int b = tid; b < BW; b += kThreads)
    if (sm.ge[b] == Pc && sm.gt[b] < Pc && Pc < V) sm.rows[atomicAdd(&sm.ctl[2], 1)] = b;
  __syncthreads();
  {
    const int n_ext = min(sm.ctl[2], BW);
    for (int e = wave; e < n_ext; e += kWaves) {
      const int b = sm.rows[e];
      int gt, ge;
      scan_row(logp + (int64_t)b * V, sm.cum[b], Pc, V, T, &gt, &ge);
      if (lane == 0) sm.ge[b] += ge;   // gt is 0 there: the row is below T past Pc
    }
  }
  __syncthreads();

  // beam order decides the ties: beam b takes t_b of its e_b ties
  const int need = BW - n_gt;   // >= 1
  int e_b = 0, gt_b = 0;
  if (tid < BW) {
    gt_b = sm.gt[tid];
    e_b = max(sm.ge[tid] - gt_b, 0);
  }
  int n_eq;
  const int E_b = block_scan(e_b, sm, &n_eq);
  const int t_b = min(max(need - E_b, 0), e_b);
  const int sel_b = tid < BW ? gt_b + t_b : 0;
  int n_sel;
  const int O_b = block_scan(sel_b, sm, &n_sel);
  if (tid < BW) {
    sm.off[tid] = O_b;
    sm.rows[tid] = gt_b;   // reuse: per-row count above T
  }
  if (tid == 0) {
    sm.ctl[3] = -1;   // the beam that takes only part of its ties
    sm.ctl[6] = 0;    // slots handed out in that beam's tie run
    sm.ctl[8] = 0;    // its candidates equal to the token threshold
  }
  __syncthreads();
  if (tid < BW && t_b > 0 && t_b < e_b) {
    sm.ctl[3] = tid;
    sm.ctl[4] = t_b;
    sm.ctl[5] = e_b;
  }
  __syncthreads();
  const int pb = sm.ctl[3];

  // 6a. winners above T and whole tie runs: one slot per thread
  for (int s = tid; s < BW; s += kThreads) {
    // the row whose output range holds slot s
    int l = 0, h = BW - 1;
    while (l < h) {
      const int m = (l + h + 1) >> 1;
      if (sm.off[m] <= s) l = m; else h = m - 1;
    }
    const int b = l;
    const int j = s - sm.off[b];
    if (b == pb && j >= sm.rows[b]) continue;   // a partial tie run: filled below
    const int jj = min(max(j, 0), V - 1);
    const uint32_t key = jj < c0 ? sm.s0[b * c0 + jj]
                                 : cand_key(sm.cum[b], logp[(int64_t)b * V + jj]);
    sm.sa[s] = ((uint64_t)(~key) << 32) | (uint32_t)b;
    sm.st[s] = (uint32_t)tok[(int64_t)b * V + jj] ^ 0x80000000u;
  }
  // 6b. the partial tie run: its t smallest token ids
  if (pb >= 0) {
    const int t = sm.ctl[4], e = sm.ctl[5];
    const int j0 = sm.rows[pb];
    const int32_t *trow = tok + (int64_t)pb * V + j0;
    uint32_t tlo = 0xffffffffu, thi = 0u;
    for (int i = tid; i < e; i += kThreads) {
      const uint32_t x = ~((uint32_t)trow[i] ^ 0x80000000u);   // larger = smaller token
      tlo = min(tlo, x);
      thi = max(thi, x);
    }
    block_minmax(tlo, thi, sm, tlo, thi);
    int n_less;
    const uint32_t X = kth_largest(
        [&](int i) { return ~((uint32_t)trow[i] ^ 0x80000000u); }, e, t, tlo, thi, sm, &n_less);
    const int base = sm.off[pb] + j0;
    const uint32_t tkey = cand_key(sm.cum[pb], logp[(int64_t)pb * V + j0]);   // == T
    for (int i = tid; i < e; i += kThreads) {
      const uint32_t x = ~((uint32_t)trow[i] ^ 0x80000000u);
      int slot = -1;
      if (x > X) {
        slot = atomicAdd(&sm.ctl[6], 1);
      } else if (x == X) {
        const int q = atomicAdd(&sm.ctl[8], 1);
        if (q < t - n_less) slot = atomicAdd(&sm.ctl[6], 1);
      }
      if (slot >= 0 && base + slot < BW) {
        sm.sa[base + slot] = ((uint64_t)(~tkey) << 32) | (uint32_t)pb;
        sm.st[base + slot] = ~x;
      }
    }
  }
  __syncthreads();

  // 7. order the winners: bitonic network over N = next power of two >= BW
  int N = 1;
  while (N < BW) N <<= 1;
  uint64_t ka = ~0ull;
  uint32_t kt = ~0u;
  if (tid < BW) {
    ka = sm.sa[tid];
    kt = sm.st[tid];
  }
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j >= 1; j >>= 1) {
      uint64_t pa;
      uint32_t pt;
      if (j >= 64) {
        __syncthreads();
        if (tid < N) {
          sm.sa[tid] = ka;
          sm.st[tid] = kt;
        }
        __syncthreads();
        const int p = (tid ^ j) & (kMaxBW - 1);
        pa = sm.sa[p];
        pt = sm.st[p];
      } else {
        const uint32_t plo = (uint32_t)__shfl_xor((int)(uint32_t)ka, j);
        const uint32_t phi = (uint32_t)__shfl_xor((int)(uint32_t)(ka >> 32), j);
        pa = ((uint64_t)phi << 32) | plo;
        pt = (uint32_t)__shfl_xor((int)kt, j);
      }
      const bool p_less = pa < ka || (pa == ka && pt < kt);
      const bool asc = (tid & k) == 0;
      const bool lower = (tid & j) == 0;
      // the lower index of a pair keeps the smaller item in an ascending run
      const bool take = (lower == asc) ? p_less : !p_less && (pa != ka || pt != kt);
      if (take) {
        ka = pa;
        kt = pt;
      }
    }
  }

  // 8. write
  if (tid < BW) {
    const int64_t o = (int64_t)r * a.out_stride + tid;
    a.score[o] = key_score(~(uint32_t)(ka >> 32));
    a.parent[o] = (int32_t)(ka & 0xffffu);
    a.token[o] = (int32_t)(kt ^ 0x80000000u);
  }
}

}  // namespace

int beam_topk_sample_len(int32_t BW, int32_t V) {
  const int c = kSampleCap / BW;
  return V < c ? V : c;
}

hipError_t launch_beam_topk(const float *cum, const float *logp, const int32_t *tok, int32_t R,
                            int32_t BW, int32_t V, float *score, int32_t *parent, int32_t *token,
                            int64_t out_stride, hipStream_t stream, LaunchEvents ev) {
  TopkArgs a{cum, logp, tok, score, parent, token, out_stride, BW, V, beam_topk_sample_len(BW, V)};
  if (ev.start)
    hipExtLaunchKernelGGL(beam_topk_kernel, dim3((unsigned)R), dim3(kThreads), 0u, stream,
                          ev.start, ev.stop, 0u, a);
  else
    hipLaunchKernelGGL(beam_topk_kernel, dim3((unsigned)R), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace xattn
