// Valid-path constraint of beam search (xGR summary, section 2.2, xBeam):
// beams may only extend along token paths of a pre-built vocabulary of valid
// items.  Masks for the early decode steps, which have many candidates, are
// dense and pre-generated; later steps, with few candidates each, keep them
// sparse.
//
// Tables.  The items form a trie.  Nodes at depth d are the distinct
// prefixes of length d, numbered in lexicographic order (the root is node 0
// of depth 0).  For every depth d < L the edges to depth d + 1 are stored as
// CSR: row_ptr[d][n] .. row_ptr[d][n+1] are the edges of node n, child_tok
// holds their tokens in ascending order, and an edge's index is the id of
// the child node it leads to.  Depths below dense_levels also get a dense bit
// row per node (bit j set iff token j is a child).  trie_build lays all of it
// out in one caller-provided host buffer; the caller copies it to the device.
//
// Kernels.  valid_mask_kernel masks one logits row per workgroup in place:
// the row's bitmap, in LDS, is the node's dense bit row (early depths) or is
// built from the node's children (later depths), and only invalid entries are
// written (-inf); valid ones are neither read nor written.  trie_advance_kernel moves
// every new beam to the child of its parent's node through its new token
// (-1 when the path leaves the vocabulary).
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

#include "xattn_internal.h"

namespace xattn {
namespace {

// masked logits are written once, past the caches (non-temporal stores)
constexpr int kMaskThreads = 256;
constexpr int kAdvanceThreads = 256;

__device__ inline const int32_t *i32_at(const uint8_t *base, int64_t off) {
  return reinterpret_cast<const int32_t *>(base + off);
}

__global__ __launch_bounds__(kMaskThreads) void valid_mask_kernel(MaskParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t bits[kMaxMaskWords];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int V = p.V, words = p.words;
  float *lg = p.logits + row * p.row_stride;
  const int n = p.node[row];
  const bool dead = n < 0 || n >= p.n_nodes;

  const uint32_t *mrow;
  if (dead) {
    for (int w = tid; w < words; w += kMaskThreads) bits[w] = 0u;
    __syncthreads();
    mrow = bits;
  } else if (p.dense) {
    // the node's dense row into LDS with one coalesced load per thread, so
    // the groups below test bits without a global round trip each; a row
    // with every bit set (every next token valid, as at a root whose
    // children cover the vocabulary) has nothing to write
    const uint32_t *src = reinterpret_cast<const uint32_t *>(p.table + p.mask_off) +
                          (int64_t)n * words;
    uint32_t all = 0xFFFFFFFFu;
    for (int w = tid; w < words; w += kMaskThreads) {
      const uint32_t x = src[w];
      bits[w] = x;
      all &= x;
    }
    if (__syncthreads_and(all == 0xFFFFFFFFu)) return;
    mrow = bits;
  } else {
    for (int w = tid; w < words; w += kMaskThreads) bits[w] = 0u;
    __syncthreads();
    const int32_t *rp = i32_at(p.table, p.row_ptr_off);
    const int32_t *ct = i32_at(p.table, p.child_tok_off);
    const int e0 = max(rp[n], 0), e1 = min(rp[n + 1], p.n_edges);
    for (int e = e0 + tid; e < e1; e += kMaskThreads) {
      const int tok = ct[e];
      if (tok >= 0 && tok < V) atomicOr(&bits[tok >> 5], 1u << (tok & 31));
    }
    __syncthreads();
    mrow = bits;
  }

  // A wave takes blocks of 256 logits: it reads the block's 8 bitmap words
  // (two broadcast 16-byte LDS reads), skips the block when all are valid,
  // and otherwise writes it with four stores of one logit per lane (64
  // consecutive logits, 256 bytes each) issued for the invalid lanes alone.
  // Valid logits are neither read nor written: the bytes written are
  // exactly the -inf entries.
  const float ninf = -INFINITY;
  const int lane = tid & 63, hi = lane >> 5, bit = lane & 31;
  const int n256 = V >> 8;
  for (int blk = tid >> 6; blk < n256; blk += kMaskThreads / 64) {
    const uint4 w0 = *reinterpret_cast<const uint4 *>(mrow + blk * 8);
    const uint4 w1 = *reinterpret_cast<const uint4 *>(mrow + blk * 8 + 4);
    if ((w0.x & w0.y & w0.z & w0.w & w1.x & w1.y & w1.z & w1.w) == 0xFFFFFFFFu) continue;
    const uint32_t wd[4] = {hi ? w0.y : w0.x, hi ? w0.w : w0.z, hi ? w1.y : w1.x,
                            hi ? w1.w : w1.z};
    float *dst = lg + (int64_t)blk * 256 + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!((wd[q] >> bit) & 1u)) __builtin_nontemporal_store(ninf, dst + 64 * q);
  }
  for (int j = (n256 << 8) + tid; j < V; j += kMaskThreads)
    if (!((mrow[j >> 5] >> (j & 31)) & 1u)) __builtin_nontemporal_store(ninf, lg + j);
}

__global__ __launch_bounds__(kAdvanceThreads) void trie_advance_kernel(AdvanceParams p) {
  const int64_t i = (int64_t)blockIdx.x * kAdvanceThreads + threadIdx.x;
  if (i >= (int64_t)p.R * p.BW) return;
  const int64_t r = i / p.BW;
  const int b = (int)(i - r * p.BW);
  const int par = min(max(p.parent[r * p.parent_stride + b], 0), p.BW - 1);
  const int n = p.node[r * p.BW + par];
  const int tok = p.token[r * p.token_stride + b];
  int out = -1;
  if (n >= 0 && n < p.n_nodes && tok >= 0 && tok < p.V) {
    const int32_t *rp = i32_at(p.table, p.row_ptr_off);
    const int32_t *ct = i32_at(p.table, p.child_tok_off);
    const int e1 = min(rp[n + 1], p.n_edges);
    int lo = max(rp[n], 0), hi = e1;   // lower bound of tok among the sorted children
    while (lo < hi) {
      const int m = (lo + hi) >> 1;
      if (ct[m] < tok) lo = m + 1; else hi = m;
    }
    if (lo < e1 && ct[lo] == tok) out = lo;
  }
  p.new_node[r * p.BW + b] = out;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

hipError_t launch_valid_mask(const MaskParams &p, hipStream_t stream, LaunchEvents ev) {
  const int64_t grid = (int64_t)p.R * p.BW;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff || p.words > kMaxMaskWords) return hipErrorInvalidConfiguration;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(valid_mask_kernel, dim3((unsigned)grid), dim3(kMaskThreads), 0u, stream,
                          ev.start, ev.stop, 0u, p);
  else
    hipLaunchKernelGGL(valid_mask_kernel, dim3((unsigned)grid), dim3(kMaskThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_trie_advance(const AdvanceParams &p, hipStream_t stream) {
  const int64_t n = (int64_t)p.R * p.BW;
  if (n == 0) return hipSuccess;
  const int64_t grid = (n + kAdvanceThreads - 1) / kAdvanceThreads;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(trie_advance_kernel, dim3((unsigned)grid), dim3(kAdvanceThreads), 0, stream,
                     p);
  return hipGetLastError();
}

const char *build_trie(const int32_t *items, int64_t n_items, int32_t levels, int32_t vocab,
                       int32_t dense_levels, TrieLayout *lay, void *host_table,
                       size_t host_bytes) {
  if (levels < 1 || levels > kMaxTrieLevels) return "levels must be in [1, 8]";
  if (vocab < 1 || vocab > 32 * kMaxMaskWords) return "vocab must be in [1, 65536]";
  if (dense_levels < 0 || dense_levels > levels) return "dense_levels must be in [0, levels]";
  if (n_items < 0 || n_items > 0x7fffffff) return "n_items must be in [0, 2^31)";
  if (n_items > 0 && !items) return "items is NULL";
  const int L = levels;
  for (int64_t i = 0; i < n_items * L; ++i)
    if (items[i] < 0 || items[i] >= vocab) return "an item token is outside [0, vocab)";

  // items in lexicographic order, duplicates next to each other
  std::vector<int32_t> order((size_t)n_items);
  std::iota(order.begin(), order.end(), 0);
  auto row = [&](int32_t i) { return items + (int64_t)i * L; };
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return std::lexicographical_compare(row(a), row(a) + L, row(b), row(b) + L);
  });
  // first position where each item differs from the previous one (L: a duplicate)
  std::vector<int8_t> first_diff((size_t)n_items);
  for (int64_t i = 0; i < n_items; ++i) {
    int f = 0;
    if (i > 0) {
      const int32_t *a = row(order[i - 1]), *b = row(order[i]);
      while (f < L && a[f] == b[f]) ++f;
    }
    first_diff[i] = (int8_t)f;
  }

  std::memset(lay, 0, sizeof(*lay));
  lay->vocab = vocab;
  lay->levels = L;
  lay->dense_levels = dense_levels;
  lay->words = (vocab + 31) / 32;
  lay->nodes[0] = 1;
  for (int64_t i = 0; i < n_items; ++i)
    for (int d = first_diff[i]; d < L; ++d) ++lay->nodes[d + 1];
  int64_t off = align256(256);   // the first 256 bytes stay free
  for (int d = 0; d < L; ++d) {
    lay->row_ptr_off[d] = off;
    off = align256(off + 4 * ((int64_t)lay->nodes[d] + 1));
    lay->child_tok_off[d] = off;
    off = align256(off + 4 * (int64_t)lay->nodes[d + 1]);
  }
  for (int d = 0; d < dense_levels; ++d) {
    lay->mask_off[d] = off;
    off = align256(off + 4 * (int64_t)lay->nodes[d] * lay->words);
  }
  lay->total_bytes = off;
  if (!host_table) return nullptr;
  if (host_bytes < (size_t)off) return "host_bytes is smaller than the layout's total_bytes";

  uint8_t *t = static_cast<uint8_t *>(host_table);
  std::memset(t, 0, (size_t)off);
  auto I = [&](int64_t o) { return reinterpret_cast<int32_t *>(t + o); };
  int32_t count[kMaxTrieLevels] = {0};   // edges created so far per depth
  I(lay->row_ptr_off[0])[0] = 0;
  for (int64_t i = 0; i < n_items; ++i) {
    const int32_t *it = row(order[i]);
    for (int d = first_diff[i]; d < L; ++d) {
      const int32_t e = count[d]++;
      I(lay->child_tok_off[d])[e] = it[d];
      if (d + 1 < L) I(lay->row_ptr_off[d + 1])[e] = count[d + 1];   // node e's first edge
    }
  }
  for (int d = 0; d < L; ++d) I(lay->row_ptr_off[d])[lay->nodes[d]] = count[d];
  for (int d = 0; d < dense_levels; ++d) {
    const int32_t *rp = I(lay->row_ptr_off[d]);
    const int32_t *ct = I(lay->child_tok_off[d]);
    uint32_t *m = reinterpret_cast<uint32_t *>(t + lay->mask_off[d]);
    for (int32_t n = 0; n < lay->nodes[d]; ++n)
      for (int32_t e = rp[n]; e < rp[n + 1]; ++e)
        m[(int64_t)n * lay->words + (ct[e] >> 5)] |= 1u << (ct[e] & 31);
  }
  return nullptr;
}

}  // namespace xattn
