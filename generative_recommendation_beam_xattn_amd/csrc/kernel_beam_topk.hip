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
constexpr int kSortCap = 1024;      // candidates the short-prefix path sorts outright
constexpr int kShortSample = 4096;  // keys of the short prefixes
constexpr int kExtStage = 32;       // scanned rows whose first chunk is kept in LDS
constexpr int kDigitBits = 9;       // radix digit width
constexpr int kRankBucketMax = 48;  // largest bucket ranked by counting
constexpr int kBins = 1 << kDigitBits;
constexpr int kMaxBW = kMaxTopkBeams;

struct TopkArgs {
  const float *cum;      // [R][BW]
  const float *logp;     // [R][BW][V]
  const int32_t *tok;    // [R][BW][V]
  float *score;          // [R] rows of BW, stride out_stride
  int32_t *parent;
  int32_t *token;
  int64_t out_stride;
  int32_t BW, V, c0, c1;
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
  uint64_t sa[kSortCap];     // sort items: (~key) << 32 | beam
  uint32_t st[kSortCap];     //             token ^ 0x80000000
  uint32_t hist[3][kBins];   // radix histograms, used in rotation; the
                             // bucket sort borrows them afterwards
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

// min and max over the block (the barrier inside also publishes the
// caller's earlier LDS stores)
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
  // no trailing barrier: every caller passes a barrier before red is
  // written again
}

// Exclusive prefix sum of v over the block's threads in order; returns this
// thread's prefix, *total the sum of v and *u_total the sum of u.
__device__ int block_scan(int v, Smem &sm, int *total, int u = 0, int *u_total = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  u = wave_sum(u);
  if (lane == 63) sm.red[wave] = inc;
  if (lane == 0) sm.red[kWaves + wave] = u;
  __syncthreads();
  int before = 0, all = 0, uall = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int x = sm.red[w];
    before += w < wave ? x : 0;
    all += x;
    uall += sm.red[kWaves + w];
  }
  __syncthreads();
  *total = all;
  if (u_total) *u_total = uall;
  return before + inc - v;
}

// Suffix sums of the kBins counts h[] (bins above each one), computed by
// every wave on its own: lane l holds bins 8l..8l+7 in c[] and, in above,
// the count of all bins of higher lanes.
__device__ inline void bins_suffix(const uint32_t *h, uint32_t c[8], uint32_t &above) {
  const int lane = threadIdx.x & 63;
  const uint4 v0 = *reinterpret_cast<const uint4 *>(h + 8 * lane);
  const uint4 v1 = *reinterpret_cast<const uint4 *>(h + 8 * lane + 4);
  c[0] = v0.x; c[1] = v0.y; c[2] = v0.z; c[3] = v0.w;
  c[4] = v1.x; c[5] = v1.y; c[6] = v1.z; c[7] = v1.w;
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) sum += c[e];
  uint32_t inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_down((int)inc, o);
    if (lane + o < 64) inc += t;
  }
  above = inc - sum;
}

// The k-th largest (1 <= k <= n) of keys get(0..n-1), all in [lo, hi], by
// most-significant-digit radix selection (9-bit digits) over the bits below
// the common prefix of lo and hi.  Every thread of the block calls it and
// gets the result; *n_above = keys strictly greater than it.
//
// One barrier per digit: after it every wave reads the whole histogram and
// finds the digit itself.  The histograms rotate through three buffers --
// pass p counts into hist[(h0 + p) % 3] and clears hist[(h0 + p + 2) % 3],
// whose last reader finished before this pass's barrier and whose next
// writer starts after the next one -- and *hsel carries h0 from call to
// call (hist[h0] and hist[(h0 + 1) % 3] are zero on entry and again on
// return).
//
// With max_passes set, selection stops after that many digits and returns
// the smallest key of the bin reached (its lower bits zero): a lower bound
// of the k-th largest with at least k keys at or above it (*n_above is then
// not meaningful).
template <class Get>
__device__ uint32_t kth_largest(Get get, int n, int k, uint32_t lo, uint32_t hi, Smem &sm,
                                int *hsel, int *n_above, int max_passes = 32) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (lo == hi) {
    *n_above = 0;
    return lo;
  }
  int bit = 32 - __clz(lo ^ hi);   // bits [0, bit) differ somewhere
  uint32_t mask = bit == 32 ? 0u : ~((1u << bit) - 1u);
  uint32_t prefix = hi & mask;
  int krem = k;
  int hs = *hsel;
  for (int pass = 0; bit > 0 && pass < max_passes; ++pass) {
    const int w = bit < kDigitBits ? bit : kDigitBits;
    const int shift = bit - w;
    const uint32_t dmask = (1u << w) - 1u;
    uint32_t *h = sm.hist[hs];
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = get(i);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    uint32_t c[8], above;
    bins_suffix(h, c, above);
    int found = -1;
    uint32_t rem = 0;
#pragma unroll
    for (int e = 7; e >= 0; --e) {
      if (above < (uint32_t)krem && above + c[e] >= (uint32_t)krem) {
        found = 8 * lane + e;
        rem = (uint32_t)krem - above;
      }
      above += c[e];
    }
    const uint64_t fm = __ballot(found >= 0);
    const int src = fm ? (int)__ffsll((unsigned long long)fm) - 1 : 0;
    const uint32_t d = (uint32_t)__shfl(found, src);
    krem = (int)__shfl((int)rem, src);
    uint32_t *g = sm.hist[hs >= 1 ? hs - 1 : 2];   // (hs + 2) % 3
    for (int i = tid; i < kBins; i += kThreads) g[i] = 0u;
    prefix |= (d & dmask) << shift;
    mask |= dmask << shift;
    bit = shift;
    hs = hs == 2 ? 0 : hs + 1;
  }
  *hsel = hs;
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


// Bitonic network over the items held by threads 0..N-1 (N a power of two,
// at most kSortCap; other threads pass the largest item), ascending in
// ((~key) << 32 | beam, token ^ 0x80000000), i.e. best candidate first;
// stages within a wave exchange through shuffles, wider ones through LDS.
// Threads 0..BW-1 then write output slot tid of request r.
__device__ void sort_and_write(uint64_t ka, uint32_t kt, int N, const TopkArgs &a, int r,
                               Smem &sm) {
  const int tid = threadIdx.x;
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
        const int p = (tid ^ j) & (kSortCap - 1);
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
  if (tid < a.BW) {
    const int64_t o = (int64_t)r * a.out_stride + tid;
    a.score[o] = key_score(~(uint32_t)(ka >> 32));
    a.parent[o] = (int32_t)(ka & 0xffffu);
    a.token[o] = (int32_t)(kt ^ 0x80000000u);
  }
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

  // Short-prefix path.  T1 = the BW-th largest of the first c1 candidates of
  // every row is a lower bound of T; every candidate at or above T1 is
  // gathered and the gathered set is sorted outright, which orders the
  // winners and applies the tie rule in one network.  It applies when at
  // most kSortCap candidates reach T1 and no row's run at or above T1
  // reaches position Pc1 (past it, uncounted candidates could still tie T).
  //
  // LDS use of s0: keys of the prefixes at [0, 4096) and their tokens at
  // [4096, 8192), both position-major (j * BW + b, swizzled below) so that
  // the lanes of a wave hold different rows and spread over the histogram
  // bins; then the
  // first scanned chunk of up to kExtStage rows: keys at [8192, 10240),
  // tokens at [10240, 12288).
  int hsel = 0;
  {
    const int c1 = a.c1;
    const int Pc1 = max(c1, P);
    const int n1 = BW * c1;
    uint32_t *skey = sm.s0;
    uint32_t *stok = sm.s0 + kShortSample;
    uint32_t *xkey = sm.s0 + 2 * kShortSample;
    uint32_t *xtok = xkey + kExtStage * 64;
    constexpr int kPer = kShortSample / kThreads;
    // slot of (row b, position j): j * BW + (b ^ (j & swz)); the XOR keeps
    // the lanes that store one row's positions on different LDS banks and
    // only permutes entries inside a position's BW slots
    const int swz = (BW & 31) == 0 ? 31 : 0;
    for (int i = tid; i < kBins; i += kThreads) {
      sm.hist[0][i] = 0u;
      sm.hist[1][i] = 0u;
      sm.hist[2][i] = 0u;
    }
    if (tid == 0) sm.ctl[2] = 0;
    // one round trip: every load of the prefixes is issued before any use
    const float cum_t = cum[tid < BW ? tid : 0];
    float cv[kPer], lv[kPer];
    int32_t tv[kPer];
    int bj[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kThreads;
      const int bb = i / c1, jj = i - bb * c1;
      bj[u] = jj * BW + (bb ^ (jj & swz));
      const int ii = i < n1 ? i : 0;
      const int bc = ii / c1, jc = ii - bc * c1;
      cv[u] = cum[bc];
      lv[u] = logp[(int64_t)bc * V + jc];
      tv[u] = tok[(int64_t)bc * V + jc];
    }
    if (tid < BW) sm.cum[tid] = cum_t;
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (tid + u * kThreads < n1) {
        const uint32_t key = cand_key(cv[u], lv[u]);
        skey[bj[u]] = key;
        stok[bj[u]] = (uint32_t)tv[u];
        lo = min(lo, key);
        hi = max(hi, key);
      }
    }
    block_minmax(lo, hi, sm, lo, hi);
    int above1;
    // one radix digit suffices: the lower edge of the bin that holds the
    // BW-th largest sampled key is itself a lower bound of T
    const uint32_t T1 = kth_largest([&](int i) { return skey[i]; }, n1, BW, lo, hi, sm, &hsel,
                                    &above1, 1);
    if (tid < BW) {
      int l = 0, h = c1;
      while (l < h) {
        const int m = (l + h) >> 1;
        if (skey[m * BW + (tid ^ (m & swz))] >= T1) l = m + 1; else h = m;
      }
      sm.ge[tid] = l;
      sm.gt[tid] = -1;   // staging slot of the row's scanned chunk, if any
      if (l == c1 && c1 < Pc1) sm.rows[atomicAdd(&sm.ctl[2], 1)] = tid;
    }
    __syncthreads();
    {
      // rows whose prefix is all >= T1 read on, 64 at a time, up to Pc1
      const int n_ext = min(sm.ctl[2], BW);
      for (int e = wave; e < n_ext; e += kWaves) {
        const int b = sm.rows[e];
        const float *lp = logp + (int64_t)b * V;
        const int32_t *tk = tok + (int64_t)b * V;
        const float cb = sm.cum[b];
        int ge = 0;
        for (int j0 = c1; j0 < Pc1; j0 += 64) {
          const int j = j0 + lane;
          const bool in = j < Pc1;
          const uint32_t key = in ? cand_key(cb, lp[j]) : 0u;
          if (j0 == c1 && e < kExtStage) {
            xkey[e * 64 + lane] = key;
            xtok[e * 64 + lane] = in ? (uint32_t)tk[j] : 0u;
          }
          const uint64_t bge = __ballot(in && key >= T1);
          ge += __popcll(bge);
          const int valid = min(64, Pc1 - j0);
          if (bge != (valid == 64 ? ~0ull : ((1ull << valid) - 1ull))) break;
        }
        if (lane == 0) {
          sm.ge[b] += ge;
          if (e < kExtStage) sm.gt[b] = e;
        }
      }
    }
    __syncthreads();
    const int ge_b = tid < BW ? sm.ge[tid] : 0;
    int n_ge, n_past;
    const int my = block_scan(ge_b, sm, &n_ge, tid < BW && ge_b == Pc1 && Pc1 < V ? 1 : 0,
                              &n_past);
    if (n_ge <= kSortCap && n_past == 0) {
      if (tid < BW) sm.off[tid] = my;
      __syncthreads();
      // gather: thread t < n_ge takes the t-th candidate at or above T1
      // (rows in order, each row's run in order), and counts it into a
      // bucket by its key's leading bits below the common prefix of T1 and
      // the largest key (a row head, so in the prefixes); larger keys take
      // lower buckets
      // bucket counts and fill levels in the two zeroed histograms, first
      // slots in the third
      uint32_t *bcnt = sm.hist[hsel];
      uint32_t *bfill = sm.hist[hsel == 2 ? 0 : hsel + 1];
      uint32_t *bbase = sm.hist[hsel == 0 ? 2 : hsel - 1];
      const int bbit = T1 == hi ? 0 : 32 - __clz(T1 ^ hi);
      const int bshift = bbit > kDigitBits ? bbit - kDigitBits : 0;
      uint64_t ka = ~0ull;
      uint32_t kt = ~0u;
      int q = 0;
      if (tid < n_ge) {
        int l = 0, h = BW - 1;
        while (l < h) {
          const int m = (l + h + 1) >> 1;
          if (sm.off[m] <= tid) l = m; else h = m - 1;
        }
        const int b = l;
        const int j = min(max(tid - sm.off[b], 0), V - 1);
        const int e = sm.gt[b];
        uint32_t key, tk;
        if (j < c1) {
          key = skey[j * BW + (b ^ (j & swz))];
          tk = stok[j * BW + (b ^ (j & swz))];
        } else if (e >= 0 && j < c1 + 64) {
          key = xkey[e * 64 + (j - c1)];
          tk = xtok[e * 64 + (j - c1)];
        } else {
          key = cand_key(sm.cum[b], logp[(int64_t)b * V + j]);
          tk = (uint32_t)tok[(int64_t)b * V + j];
        }
        ka = ((uint64_t)(~key) << 32) | (uint32_t)b;
        kt = tk ^ 0x80000000u;
        q = (int)min((hi >> bshift) - (max(key, T1) >> bshift), (uint32_t)(kBins - 1));
        atomicAdd(&bcnt[q], 1u);
      }
      __syncthreads();
      // first slot of every bucket: each wave computes the prefix sums and
      // stores them (all waves store the same values, and each wave reads
      // only after its own stores)
      {
        uint32_t c[8], above;
        bins_suffix(bcnt, c, above);   // counts of higher lanes' bins...
        // a crowded bucket (many equal keys) would make the ranking below
        // quadratic: sort the gathered set with the bitonic network instead
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, c[e]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
        if (m > kRankBucketMax) {
          int N = 1;
          while (N < n_ge) N <<= 1;
          sort_and_write(ka, kt, N, a, r, sm);
          return;
        }
        // ...but buckets run upwards: exclusive prefix = total - above - own
        uint32_t total = above;
#pragma unroll
        for (int e = 0; e < 8; ++e) total += c[e];
        total = (uint32_t)__shfl((int)total, 0);
        uint32_t run = total - above;
#pragma unroll
        for (int e = 7; e >= 0; --e) {
          run -= c[e];
          bbase[8 * lane + e] = run;
        }
      }
      int slot = -1;
      if (tid < n_ge) {
        slot = (int)(bbase[q] + atomicAdd(&bfill[q], 1u));
        sm.sa[slot] = ka;
        sm.st[slot] = kt;
      }
      __syncthreads();
      // rank inside the bucket by the full order; the first BW ranks are the
      // output
      if (tid < n_ge) {
        const int b0 = (int)bbase[q], b1 = b0 + (int)bcnt[q];
        int rank = b0;
#pragma unroll 4
        for (int i = b0; i < b1; ++i) {
          const uint64_t ya = sm.sa[i];
          const uint32_t yt = sm.st[i];
          rank += (ya < ka || (ya == ka && yt < kt) || (ya == ka && yt == kt && i < slot)) ? 1 : 0;
        }
        if (rank < BW) {
          const int64_t o = (int64_t)r * a.out_stride + rank;
          a.score[o] = key_score(~(uint32_t)(ka >> 32));
          a.parent[o] = (int32_t)(ka & 0xffffu);
          a.token[o] = (int32_t)(kt ^ 0x80000000u);
        }
      }
      return;
    }
  }

  // General path, taken when the short prefixes leave too many candidates or
  // a run that may continue past the counted prefix.
  for (int b = tid; b < BW; b += kThreads) {
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
  const uint32_t T0 =
      kth_largest([&](int i) { return sm.s0[i]; }, n0, BW, lo, hi, sm, &hsel, &above0);

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
    T = kth_largest([&](int i) { return sm.lkey[i]; }, n_list, BW, llo, lhi, sm, &hsel, &above);
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
        [&](int i) { return ~((uint32_t)trow[i] ^ 0x80000000u); }, e, t, tlo, thi, sm, &hsel,
        &n_less);
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

  // 7. order the winners and write them
  int N = 1;
  while (N < BW) N <<= 1;
  sort_and_write(tid < BW ? sm.sa[tid] : ~0ull, tid < BW ? sm.st[tid] : ~0u, N, a, r, sm);
}

}  // namespace

int beam_topk_sample_len(int32_t BW, int32_t V) {
  const int c = kSampleCap / BW;
  return V < c ? V : c;
}

// Short prefix: 4096 / BW candidates per row (8 at BW = 512, 32 at 128).
static int beam_topk_short_len(int32_t BW, int32_t V) {
  const int c = kShortSample / BW;
  return V < c ? V : c;
}

hipError_t launch_beam_topk(const float *cum, const float *logp, const int32_t *tok, int32_t R,
                            int32_t BW, int32_t V, float *score, int32_t *parent, int32_t *token,
                            int64_t out_stride, hipStream_t stream, LaunchEvents ev) {
  TopkArgs a{cum, logp, tok, score, parent, token, out_stride, BW, V,
             beam_topk_sample_len(BW, V), beam_topk_short_len(BW, V)};
  static_assert(kMaxBW * 8 <= kShortSample && kShortSample <= kSampleCap, "short sample size");
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(beam_topk_kernel, dim3((unsigned)R), dim3(kThreads), 0u, stream,
                          ev.start, ev.stop, 0u, a);
  else
    hipLaunchKernelGGL(beam_topk_kernel, dim3((unsigned)R), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace xattn
