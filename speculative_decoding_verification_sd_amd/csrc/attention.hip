// Verify attention on gfx950.
//
// Speculation raises the attention GEMM-M from G to G*(1+D): every KV head
// serves the G query heads that share it at each of the 1+D verify positions,
// all over the same KV cache ("Co-Designing AI Models Using Speculative
// Decoding for Faster LLM Inference", translated page, section "Draft length
// and attention performance").  The kernel therefore treats one (sequence,
// KV head) as a dense [R = G*(1+D_b)] x [d] query block and streams the
// sequence's pages once.  Position i of the block sees keys up to its own
// absolute position N-(1+D_b)+i (causal inside the block).
//
// Work decomposition (split-KV).  A sequence's keys are cut into chunks of
// `chunk` keys; a work item is (sequence, KV head, chunk).  A one-workgroup
// plan kernel picks the chunk (a multiple of 64 keys) from a bound on the
// schedule's length, lists the items longest first and writes one descriptor
// per item; a persistent grid walks the list.
//
// Per item, a workgroup runs over 32-key tiles (two 16-key pages):
//   * K and V tiles travel global -> LDS with global_load_lds_dwordx4 (no
//     registers) into a ring of tiles, paced by explicit vmcnt waits and a bare
//     s_barrier.  K pages are key-major and V pages d-major ([d][16 keys]);
//     LDS rows are XOR-swizzled in 16-byte chunks against bank conflicts.
//   * S^T = K * Q^T with Q held in registers, so each lane holds one query row
//     and the row reductions stay within a lane pair (v_permlane32_swap).
//     verify_attn_wide (more than 64 rows) uses v_mfma_f32_32x32x16_bf16 with
//     8 waves in two sets that take alternate tiles or row blocks (and, from
//     129 to 144 rows, one 16-row block of 16x16x32 MFMAs for the rows past
//     128); verify_attn_main (up to 64 rows) uses v_mfma_f32_16x16x32_bf16.
//   * Softmax: each row's reference max is fixed by the item's first tile, so
//     later tiles need neither a row max nor a rescale; an item whose row sum
//     ends above 2^64 (a score far above its reference) is computed again with
//     a running max.
//   * P (bf16) is taken straight from the S^T accumulators as the B operand of
//     O^T = V^T * P^T, and V^T comes from the d-major pages with ds_read_b128.
// Items that cover a whole sequence write the output; otherwise the
// unnormalised partial (O, m, l) goes to the workspace and a combine kernel
// merges the splits with their log-sum-exp weights.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace sdv {

constexpr int kPage = 16;
constexpr int kMinChunk = 256;
constexpr int kMaxChunk = 32768;         // keys per work item; bounds the per-item page list in LDS
constexpr int kPlanThreads = 256;
constexpr int kItemsPerSlot = 4;         // work items per resident workgroup the workspace admits
constexpr int kItemOverheadBytes = 192 * 1024;   // an item's fixed cost (set-up, partials) in bytes of K/V
constexpr int kPlanHeader = 16;

// LDS operands the row-split step reads ahead of their MFMAs.  Build-time tunable.
#ifndef SDV_RS_AHEAD
#define SDV_RS_AHEAD 2
#endif

// LDS bytes of the K/V rings of one CU (at most 8 tiles per workgroup),
// shared by its resident workgroups.  Build-time tunable.
#ifndef SDV_RING_BYTES_PER_CU
#define SDV_RING_BYTES_PER_CU 131072
#endif

struct ItemDesc {
  int b, h, k_begin, k_end;   // sequence, KV head, key range of this split
  int t0, D, N, nsplit;       // first verify row, drafts, keys, splits of the sequence
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int* block_table;
  const int* kv_len;
  const int* q_start;
  void* out;
  float* part_o;    // [item_cap, rpad, d]   unnormalised partial outputs
  float* part_ml;   // [item_cap, rpad, 2]   (running max in log2 units, sum)
  int* plan;        // [16 + 3B + 1]: chunk, total items, full items, split sequences, work counters,
                    // item_start, tail_pos, split sequence list
  const unsigned long long* tmask;   // NULL: causal block; else per verify row, the nodes of its draft tree it sees
  ItemDesc* items;  // [item_cap]
  int B, Hkv, G, max_pages, num_pages, max_draft, rpad, total_q, item_cap;
  float scale_log2;
  // the plan's inputs: explicit chunk (0: chosen), resident workgroups, an
  // item's fixed cost in keys, whether the combine walks a split list; fused:
  // the main kernels make the plan themselves (small batches, no plan launch)
  int fixed_chunk, slots, ovh_keys, list_splits, fused;
};

__device__ __forceinline__ int seq_keys(const AttnParams& p, int b) {
  return min(max(p.kv_len[b], 0), p.max_pages * kPage);
}

__device__ __forceinline__ int seq_drafts(const AttnParams& p, int b) {
  return min(max(p.q_start[b + 1] - p.q_start[b] - 1, 0), p.max_draft);
}

// ---------------------------------------------------------------------------
// Draft-tree masks, one wave per sequence: node i of sequence b sees its root
// path, mask(i) = mask(parent(i)) | bit i with mask(root) = bit 0, where
// parents[(q_start[b]-b) + i-1] < i (the LLM inference handbook, section
// "Medusa": tree attention keeps the causal order inside each branch).  A
// parent out of that range is taken as the root.  Lane i holds node i and
// doubles its reach six times (pointer jumping: after round k its mask holds
// the nodes up to 2^(k+1)-1 steps above it and `up` the node 2^(k+1) steps
// above, the root's parent being the root), which covers every path of a tree
// of at most 64 nodes.
constexpr int kMaskSeqsPerBlock = 4;
__global__ __launch_bounds__(64 * kMaskSeqsPerBlock) void verify_tree_masks(AttnParams p, const int* parents,
                                                                             unsigned long long* masks) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kMaskSeqsPerBlock + (threadIdx.x >> 6);
  if (b >= p.B) return;                         // (whole waves)
  const int t0 = p.q_start[b];
  const int T = min(seq_drafts(p, b), 63);
  const int d0 = t0 - b;
  if (t0 < 0 || t0 + T >= p.total_q || d0 < 0 || d0 + T > p.total_q - p.B) return;
  int up = 0;
  if (lane >= 1 && lane <= T) {
    const int q = parents[d0 + lane - 1];
    up = (q >= 0 && q < lane) ? q : 0;
  }
  unsigned long long m = 1ull << lane;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const unsigned long long mu = __shfl(m, up);
    const int uu = __shfl(up, up);
    m |= mu;
    up = uu;
  }
  if (lane <= T) masks[t0 + lane] = m;
}

// ---------------------------------------------------------------------------
// Plan (one workgroup).
//
// Chunk: `fixed_chunk` if non-zero.  Otherwise thread t evaluates candidate
// plan_candidate(t) (at most the longest sequence, rounded up to 64, and at
// most kMaxChunk): with items(c) = Hkv * sum_b max(1, ceil(N_b / c)), the
// schedule of the persistent grid takes at least the average load per slot,
// (Hkv * sum_b N_b + ovh * items(c)) / slots keys (ovh: fixed cost of an item
// in keys), and at least the longest item, min(c, max_b N_b).  The plan takes
// the chunk with the smallest of these bounds (the largest chunk on ties)
// among those whose items fit the workspace (the smaller chunk on ties).
//
// Order: items go to the workgroups in a longest-first order, which keeps the
// tail of the schedule short when sequence lengths differ: when some items are
// shorter than the chunk and there are more items than workgroups, the grid
// takes the items after its first round from eight counters (workgroup w uses
// counter w % 8 and the items i with i % 8 == w % 8) as workgroups finish.  Every full-chunk item comes
// first; then the one shorter item of each (sequence, head), by its length in
// kLenBuckets buckets, longest bucket first.  Split-KV partials stay addressed
// by the natural index item_start[b] + h * nsplit_b + split.
//
// plan[]: [0] chunk, [1] items, [2] full-chunk items, [3] sequences split in
// more than one item (when list_splits), [8..15] work counters (cleared here),
// then from kPlanHeader on item_start[0..B], tail_pos[0..B-1] (scheduled index
// of head 0's shorter item of sequence b, -1: none), when list_splits the list
// of the split sequences (plan[3] entries, any order) for the combine of large
// batches, and full_base[0..B-1] (scheduled index of sequence b's first
// full-chunk item).  The plan kernel writes the header and the per-sequence
// tables, and the descriptors and the split list too up to kPlanWrites
// (sequence, head) pairs; beyond, verify_attn_items writes those.
constexpr int kLenBuckets = 64;
constexpr int kPlanCacheSeqs = 8192;     // sequences whose key counts the plan keeps in LDS (32 KiB)
constexpr int kHistBins = kMaxChunk / 64 + 2;   // ceil(N/64) = 0 .. 512, and "longer"
constexpr int kBinsPerLane = (kHistBins + 63) / 64;   // the suffix scan: one wave over the bins

// Chunk candidate t of the plan's search (t < kPlanThreads, increasing in t):
// every multiple of 64 keys from 256 to 15552, then 16384 .. 30720 in steps of
// 1024 and kMaxChunk itself.
__device__ __forceinline__ int plan_candidate(int t) {
  return t < 240 ? kMinChunk + 64 * t : t < kPlanThreads - 1 ? 16384 + 1024 * (t - 240) : kMaxChunk;
}
constexpr int kLongSeqs = 256;           // sequences longer than kMaxChunk the chunk search lists in LDS
constexpr int kDirectSeqs = 64;          // chunk search: batches this small skip the histogram

// floor(n / c) for 0 <= n < 2^24 and 1 <= c <= 2^24: the float quotient
// corrected to the exact one.
__device__ __forceinline__ int floor_div_keys(int n, int c, float rc) {
  int q = (int)((float)n * rc);
  if (q * c > n) --q;
  if ((q + 1) * c <= n) ++q;
  return q;
}

// atomicAdd(&s[key], 1) of every lane with `active`; returns the lane's old
// value.  When all active lanes of the wave share one key (equal lengths: one
// bucket) it is one LDS atomic for the wave, the lanes taking consecutive
// values in lane order, instead of a 64-way conflict; otherwise one atomic per
// lane, which the LDS runs in parallel over distinct keys.  Every lane of the
// wave calls it.
__device__ __forceinline__ int wave_bucket_add(int* s, int key, bool active) {
  const int lane = threadIdx.x & 63;
  const unsigned long long act = __ballot(active);
  if (!act) return 0;
  const int leader = __ffsll(act) - 1;
  const int k0 = __shfl(key, leader);
  if (__ballot(active && key == k0) == act) {
    int base = 0;
    if (lane == leader) base = atomicAdd(&s[k0], (int)__popcll(act));
    base = __shfl(base, leader);
    return active ? base + (int)__popcll(act & ((1ull << lane) - 1ull)) : 0;
  }
  return active ? atomicAdd(&s[key], 1) : 0;
}

// The descriptors of (sequence b, KV head h): its full-chunk items at
// full_base + h * full + split, its shorter item (if any) at tail_pos + h (the
// plan's scheduled positions for b); and, for the listed combine, the sequence
// in the split list when it has more than one item.
__device__ void write_item_descs(const AttnParams& p, int b, int h, int chunk, int N, int t0, int D, int full_base,
                                 int tail_pos, int list_splits) {
  int* split_list = p.plan + kPlanHeader + 2 * p.B + 1;
  const int full = N / chunk;
  const bool tail = N - full * chunk != 0 || N == 0;
  const int ns = full + (tail ? 1 : 0);
  ItemDesc d;
  d.b = b;
  d.h = h;
  d.t0 = t0;
  d.D = D;
  d.N = N;
  d.nsplit = ns;
  const int fbase = full_base + h * full;
  for (int s = 0; s < full; ++s) {
    if (fbase + s < 0 || fbase + s >= p.item_cap) break;
    d.k_begin = s * chunk;
    d.k_end = d.k_begin + chunk;
    p.items[fbase + s] = d;
  }
  if (tail) {
    const int pos = tail_pos + h;
    if (pos >= 0 && pos < p.item_cap) {
      d.k_begin = full * chunk;
      d.k_end = N;
      p.items[pos] = d;
    }
  }
  if (list_splits && h == 0 && ns > 1) split_list[atomicAdd(p.plan + 3, 1)] = b;   // (any order: each head merges alone)
}

// Up to this many (sequence, KV head) pairs the plan kernel writes the
// descriptors itself; beyond, verify_attn_items spreads them over the GPU (one
// workgroup's stores would take tens of microseconds).
constexpr int kPlanWrites = 4096;

__global__ __launch_bounds__(kPlanThreads) void verify_attn_plan(AttnParams p, int fixed_chunk, int slots,
                                                                 int ovh_keys, int list_splits) {
  __shared__ int s_bucket[kLenBuckets];
  __shared__ unsigned long long s_best;
  __shared__ long long s_ksum, s_full;
  __shared__ int s_nmax;
  __shared__ int s_n[kPlanCacheSeqs];      // N_b
  // the descriptors' fields, for the batches whose descriptors this kernel writes
  __shared__ int s_t0[kPlanWrites], s_d[kPlanWrites], s_tail[kPlanWrites], s_fbase[kPlanWrites];
  __shared__ int s_wsum[2][kPlanThreads / 64];
  __shared__ int s_hist[kHistBins];        // sequences by ceil(N/64), the last bin N > kMaxChunk
  __shared__ int s_above[kHistBins];       // s_above[x] = sequences with ceil(N/64) > x
  __shared__ int s_long[kLongSeqs];        // ceil(N/64) of the sequences longer than kMaxChunk
  __shared__ int s_nlong;
  const int tid = threadIdx.x;
  const int max_keys = p.max_pages * kPage;
  const int cap_chunk = max(kMinChunk, min(kMaxChunk, (max_keys + 63) / 64 * 64));
  const int my_chunk = min(plan_candidate(tid), cap_chunk);
  int* tail_pos = p.plan + kPlanHeader + p.B + 1;
  auto keys_of = [&](int b) { return b < kPlanCacheSeqs ? s_n[b] : seq_keys(p, b); };

  // (1) the chunk.  Candidates are c = 64 d keys (d >= 4), and ceil(N/c) =
  // ceil(ceil(N/64) / d), so with n_b = ceil(N_b/64) the item count is
  // sum_b max(1, ceil(n_b/d)) = B + sum_{k>=1} #{b : n_b > k d}.  For the
  // sequences of at most kMaxChunk keys (n_b <= 512) the terms come from the
  // suffix counts of their histogram (s_above, non-increasing, so the sum stops
  // at the first zero); each longer sequence adds ceil(n_b/d) - 1.  The search
  // costs O(B + 256 * long sequences) instead of 256 divisions per sequence.
  // Up to kDirectSeqs sequences every candidate simply divides each length.
  const bool direct = p.B <= kDirectSeqs;
  const bool writes = p.B * p.Hkv <= kPlanWrites;   // (then B <= kPlanWrites: the fields fit in LDS)
  if (tid == 0) { s_best = ~0ull; s_ksum = 0; s_full = 0; s_nmax = 0; s_nlong = 0; }
  if (tid < kLenBuckets) s_bucket[tid] = 0;
  if (!direct) {
    for (int i = tid; i < kHistBins; i += kPlanThreads) s_hist[i] = 0;
    __syncthreads();
  }
  long long my_items = 0, ksum = 0;
  int nmax = 0;
  constexpr int kLoadGroups = 4;   // groups of sequences whose loads are issued before any is used
  for (int base0 = 0; base0 < p.B; base0 += kLoadGroups * kPlanThreads) {
    int nbv[kLoadGroups], t0v[kLoadGroups], dv[kLoadGroups];
#pragma unroll
    for (int u = 0; u < kLoadGroups; ++u) {
      const int b = base0 + u * kPlanThreads + tid;
      const bool mine = b < p.B && writes;
      nbv[u] = b < p.B ? seq_keys(p, b) : 0;
      t0v[u] = mine ? p.q_start[b] : 0;
      dv[u] = mine ? seq_drafts(p, b) : 0;
    }
#pragma unroll
    for (int u = 0; u < kLoadGroups; ++u) {
      const int b = base0 + u * kPlanThreads + tid;
      const bool in = b < p.B;
      const int nb = nbv[u];
      if (b < kPlanCacheSeqs) s_n[b] = nb;
      if (in && writes) {
        s_t0[b] = t0v[u];
        s_d[b] = dv[u];
      }
      ksum += nb;
      nmax = max(nmax, nb);
      if (!direct) {   // (every lane takes part: the histogram adds are per wave and distinct bin)
        const int n64 = (nb + 63) >> 6;
        wave_bucket_add(s_hist, min(n64, kHistBins - 1), in);
        if (in && n64 > kHistBins - 2) {
          const int sl = atomicAdd(&s_nlong, 1);
          if (sl < kLongSeqs) s_long[sl] = n64;
        }
      }
    }
  }
  __syncthreads();
  static_assert(kBinsPerLane * 64 >= kHistBins, "one wave over the bins");
  static_assert(kDirectSeqs <= kPlanCacheSeqs, "the direct count reads the lengths from LDS");
  if (direct) {
    for (int b = 0; b < p.B; ++b) my_items += max(1, (s_n[b] + my_chunk - 1) / my_chunk);
  } else {
    if (tid < 64) {                                  // suffix counts: s_above[x] = short sequences past bin x
      int loc[kBinsPerLane], tot = 0;
  #pragma unroll
      for (int q = 0; q < kBinsPerLane; ++q) {
        const int x = kBinsPerLane * tid + q;
        loc[q] = x < kHistBins - 1 ? s_hist[x] : 0;   // (the last bin: the long ones)
        tot += loc[q];
      }
      int suf = tot;                                 // inclusive suffix scan over the lanes
  #pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_down(suf, off);
        if (tid + off < 64) suf += t;
      }
      int after = suf - tot;
  #pragma unroll
      for (int q = kBinsPerLane - 1; q >= 0; --q) {
        if (kBinsPerLane * tid + q < kHistBins) s_above[kBinsPerLane * tid + q] = after;
        after += loc[q];
      }
    }
    __syncthreads();
    if (s_nlong <= kLongSeqs) {
      const int d = my_chunk >> 6;
      long long acc = p.B;
      for (int x = d; x <= kHistBins - 2; x += d) {
        const int a = s_above[x];
        if (a == 0) break;
        acc += a;
      }
      for (int i = 0; i < s_nlong; ++i) acc += (s_long[i] + d - 1) / d - 1;
      my_items = acc;
    } else {
      // more long sequences than listed: count each one (the attention over that
      // many sequences of more than kMaxChunk keys takes far longer than this)
      for (int b = 0; b < p.B; ++b) my_items += max(1, (keys_of(b) + my_chunk - 1) / my_chunk);
    }
  }
  // (block reductions: a wave reduction, then one LDS atomic per wave)
  const int lane = tid & 63;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ksum += __shfl_xor(ksum, off);
    nmax = max(nmax, __shfl_xor(nmax, off));
  }
  __syncthreads();
  if (lane == 0) {
    atomicAdd((unsigned long long*)&s_ksum, (unsigned long long)ksum);
    atomicMax(&s_nmax, nmax);
  }
  __syncthreads();
  const long long items_c = my_items * p.Hkv;
  unsigned long long key = ~0ull;
  if (items_c <= p.item_cap) {
    const long long load = (s_ksum * p.Hkv + (long long)ovh_keys * items_c + slots - 1) / slots;
    const long long est = max(load, (long long)min(my_chunk, s_nmax));
    key = ((unsigned long long)est << 9) | (unsigned long long)tid;   // ties: the smaller chunk
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = min(key, (unsigned long long)__shfl_xor(key, off));
  if (lane == 0) atomicMin(&s_best, key);
  __syncthreads();
  int chunk = cap_chunk;
  if (fixed_chunk > 0) chunk = fixed_chunk;
  else if (s_best != ~0ull) chunk = min(plan_candidate((int)(s_best & 511)), cap_chunk);

  // (2) the shorter items: count per length bucket (bucket 0 = longest), and
  // the number of full-chunk items
  const float rchunk = 1.f / (float)chunk, rchunk1 = 1.f / (float)(chunk + 1);
  auto split_of = [&](int N, int& full, int& tail_len) {   // full chunks, and the shorter item's length (-1: none)
    full = floor_div_keys(N, chunk, rchunk);
    tail_len = (N - full * chunk != 0 || N == 0) ? N - full * chunk : -1;
  };
  auto bucket_of = [&](int len) {   // (len <= chunk <= kMaxChunk: the product fits 32 bits)
    return kLenBuckets - 1 - floor_div_keys(len * kLenBuckets, chunk + 1, rchunk1);
  };
  long long nfull = 0;
  for (int base = 0; base < p.B; base += kPlanThreads) {   // (uniform trip count: the bucket adds are per wave)
    const int b = base + tid;
    int full = 0, tl = -1;
    if (b < p.B) split_of(keys_of(b), full, tl);
    nfull += (long long)full * p.Hkv;
    wave_bucket_add(s_bucket, tl >= 0 ? bucket_of(tl) : 0, tl >= 0);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) nfull += __shfl_xor(nfull, off);
  if (lane == 0) atomicAdd((unsigned long long*)&s_full, (unsigned long long)nfull);
  __syncthreads();
  static_assert(kLenBuckets == 64, "one lane of wave 0 per bucket");
  if (tid < 64) {                                  // bucket counts -> exclusive prefix (running cursors)
    const int c = s_bucket[tid];
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (tid >= off) incl += t;
    }
    s_bucket[tid] = incl - c;
  }
  __syncthreads();
  for (int base = 0; base < p.B; base += kPlanThreads) {
    const int b = base + tid;
    int full = 0, tl = -1;
    if (b < p.B) split_of(keys_of(b), full, tl);
    const int slot = wave_bucket_add(s_bucket, tl >= 0 ? bucket_of(tl) : 0, tl >= 0);
    const int tp = tl >= 0 ? (int)(s_full + (long long)slot * p.Hkv) : -1;
    if (b < p.B) {
      if (writes) s_tail[b] = tp;
      else tail_pos[b] = tp;
    }
  }
  __syncthreads();

  // (3) per-sequence item starts: sequences in groups of kPlanThreads, inclusive
  // scans of the items and of the full-chunk items (within each wave by
  // shuffles, then the totals of the waves before it).  verify_attn_items
  // writes the descriptors from these tables, one thread per sequence, over
  // many workgroups.
  int* full_base = p.plan + kPlanHeader + 3 * p.B + 1;
  if (tid == 0) p.plan[3] = 0;   // split sequences, counted as their descriptors are written
  int carry = 0, fcarry = 0;
  for (int base = 0; base < p.B; base += kPlanThreads) {
    const int b = base + tid;
    int v = 0, full = 0, tl = -1;
    if (b < p.B) {
      split_of(keys_of(b), full, tl);
      v = (full + (tl >= 0 ? 1 : 0)) * p.Hkv;
    }
    int sv = v, sf = full * p.Hkv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a = __shfl_up(sv, off), f = __shfl_up(sf, off);
      if (lane >= off) { sv += a; sf += f; }
    }
    if (lane == 63) { s_wsum[0][tid >> 6] = sv; s_wsum[1][tid >> 6] = sf; }
    __syncthreads();
    for (int w = 0; w < (tid >> 6); ++w) { sv += s_wsum[0][w]; sf += s_wsum[1][w]; }
    if (b < p.B) {
      p.plan[kPlanHeader + b] = carry + sv - v;
      if (writes) {
        s_fbase[b] = fcarry + sf - full * p.Hkv;
      } else {
        full_base[b] = fcarry + sf - full * p.Hkv;
      }
    }
    if (tid == kPlanThreads - 1) { s_wsum[0][0] = carry + sv; s_wsum[1][0] = fcarry + sf; }
    __syncthreads();
    carry = s_wsum[0][0];
    fcarry = s_wsum[1][0];
    __syncthreads();
  }
  if (writes) {
    for (int idx = tid; idx < p.B * p.Hkv; idx += kPlanThreads) {
      const int b = idx / p.Hkv;
      write_item_descs(p, b, idx - b * p.Hkv, chunk, keys_of(b), s_t0[b], s_d[b], s_fbase[b], s_tail[b],
                       list_splits);
    }
  }
  if (tid < 8) p.plan[8 + tid] = 0;
  if (tid == 0) {
    p.plan[0] = chunk;
    p.plan[1] = carry;
    p.plan[2] = (int)s_full;
    p.plan[kPlanHeader + p.B] = carry;
  }
}



// The descriptors of batches with more than kPlanWrites (sequence, KV head)
// pairs, one thread per pair.
__global__ __launch_bounds__(256) void verify_attn_items(AttnParams p, int list_splits) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.B * p.Hkv) return;
  const int chunk = p.plan[0];
  if (chunk < 64) return;
  const int b = idx / p.Hkv;
  write_item_descs(p, b, idx - b * p.Hkv, chunk, seq_keys(p, b), p.q_start[b], seq_drafts(p, b),
                   p.plan[kPlanHeader + 3 * p.B + 1 + b], p.plan[kPlanHeader + p.B + 1 + b], list_splits);
}

// ---------------------------------------------------------------------------
// The plan inside the main kernels, for batches of up to kFusedSeqs sequences:
// every workgroup takes the same decisions as verify_attn_plan from the same
// inputs (the chunk by the same rule over the same candidates; full-chunk
// items first in (sequence, head, split) order, then the shorter items longest
// first by length bucket, sequences in index order within a bucket), in its own
// LDS, so the call needs no plan launch.  Workgroup w then takes item w of
// every round of gridDim items, walking the rounds in snake order (forward in
// even rounds, backward in odd ones), which pairs the longest items with the
// shortest ones, and finds each item's descriptor from the LDS tables.
// Workgroup 0 writes the plan header and the per-sequence item starts that the
// combine reads (the launch boundary orders them before it); each item's
// descriptor is written by the workgroup that takes it.
constexpr int kFusedSeqs = 32;

struct FusedPlan {
  unsigned long long best;
  int chunk, total, nfull;
  int n[kFusedSeqs], t0[kFusedSeqs], dr[kFusedSeqs], tseq[kFusedSeqs];
  int fpre[kFusedSeqs + 1];     // full-chunk items of the sequences before b (x H_kv)
  int istart[kFusedSeqs + 1];   // natural index of sequence b's first item
};

// ceil(n / c) for 0 <= n < 2^24 and 64 <= c <= kMaxChunk: the float quotient
// (relative error far below 1/n) corrected to the exact floor, then rounded up.
__device__ __forceinline__ int ceil_div_keys(int n, int c, float rc) {
  const int q = floor_div_keys(n, c, rc);
  return q + (q * c < n ? 1 : 0);
}

// All threads of the workgroup (at least kPlanThreads) call it.
__device__ void fused_plan(const AttnParams& p, FusedPlan& fp) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = p.B;
  if (tid < B) {
    fp.n[tid] = seq_keys(p, tid);
    fp.t0[tid] = p.q_start[tid];
    fp.dr[tid] = seq_drafts(p, tid);
  }
  if (tid == 0) fp.best = ~0ull;
  block_sync_lds();
  const int max_keys = p.max_pages * kPage;
  const int cap_chunk = max(kMinChunk, min(kMaxChunk, (max_keys + 63) / 64 * 64));
  int chunk = cap_chunk;
  if (p.fixed_chunk > 0) {
    chunk = p.fixed_chunk;
  } else {
    long long ksum = 0;
    int nmax = 0;
    for (int b = 0; b < B; ++b) {
      ksum += fp.n[b];
      nmax = max(nmax, fp.n[b]);
    }
    unsigned long long key = ~0ull;
    if (tid < kPlanThreads) {
      const int c = min(plan_candidate(tid), cap_chunk);
      const float rc = 1.f / (float)c;
      long long items = 0;
      for (int b = 0; b < B; ++b) items += max(1, ceil_div_keys(fp.n[b], c, rc));
      items *= p.Hkv;
      if (items <= p.item_cap) {
        const long long load = (ksum * p.Hkv + (long long)p.ovh_keys * items + p.slots - 1) / p.slots;
        const long long est = max(load, (long long)min(c, nmax));
        key = ((unsigned long long)est << 9) | (unsigned long long)tid;   // ties: the smaller chunk
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) key = min(key, (unsigned long long)__shfl_xor(key, off));
    if (lane == 0 && key != ~0ull) atomicMin(&fp.best, key);
    block_sync_lds();
    if (fp.best != ~0ull) chunk = min(plan_candidate((int)(fp.best & 511)), cap_chunk);
  }
  if (tid < 64) {   // one wave: lane b takes sequence b
    const bool in = tid < B;
    const int N = in ? fp.n[tid] : 0;
    const int full = in ? N / chunk : 0;
    const bool tail = in && (N % chunk != 0 || N == 0);
    const int bucket = tail ? kLenBuckets - 1 - ((N - full * chunk) * kLenBuckets) / (chunk + 1) : 0;
    int sf = full * p.Hkv, si = in ? (full + (tail ? 1 : 0)) * p.Hkv : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a = __shfl_up(sf, off), c = __shfl_up(si, off);
      if (lane >= off) { sf += a; si += c; }
    }
    if (in) {
      fp.fpre[tid + 1] = sf;
      fp.istart[tid + 1] = si;
    }
    int rank = 0;
    for (int b2 = 0; b2 < B; ++b2) {
      const int t2 = __shfl(tail ? 1 : 0, b2), k2 = __shfl(bucket, b2);
      if (t2 && (k2 < bucket || (k2 == bucket && b2 < tid))) ++rank;
    }
    if (tail) fp.tseq[rank] = tid;
    const int nf = __shfl(sf, max(B - 1, 0)), tot = __shfl(si, max(B - 1, 0));
    if (tid == 0) {
      fp.fpre[0] = 0;
      fp.istart[0] = 0;
      fp.chunk = chunk;
      fp.nfull = B > 0 ? nf : 0;
      fp.total = B > 0 ? tot : 0;
    }
  }
  block_sync_lds();
  if (blockIdx.x == 0) {   // what the combine reads: the header, item starts, split sequences
    int* tail_pos = p.plan + kPlanHeader + p.B + 1;
    int* split_list = p.plan + kPlanHeader + 2 * p.B + 1;
    if (tid <= B) p.plan[kPlanHeader + tid] = fp.istart[tid];
    if (tid < B) tail_pos[tid] = -1;
    if (tid < 64) {
      const bool split = tid < B && fp.istart[tid + 1] - fp.istart[tid] > p.Hkv;
      const unsigned long long m = __ballot(split);
      if (p.list_splits && split) split_list[__popcll(m & ((1ull << tid) - 1))] = tid;
      if (tid == 0) {
        p.plan[0] = fp.chunk;
        p.plan[1] = fp.total;
        p.plan[2] = fp.nfull;
        p.plan[3] = p.list_splits ? (int)__popcll(m) : 0;
      }
    }
  }
}

// Item i of the fused plan and its partial slot (natural index).
__device__ __forceinline__ ItemDesc fused_item(const AttnParams& p, const FusedPlan& fp, int i, int& pslot) {
  const int chunk = fp.chunk;
  int b, h, s, k0, k1;
  if (i < fp.nfull) {
    b = 0;
    while (b + 1 < p.B && fp.fpre[b + 1] <= i) ++b;
    const int full = max((fp.fpre[b + 1] - fp.fpre[b]) / p.Hkv, 1);
    const int r = i - fp.fpre[b];
    h = r / full;
    s = r - h * full;
    k0 = s * chunk;
    k1 = k0 + chunk;
  } else {
    const int j = i - fp.nfull;
    const int rank = j / p.Hkv;
    h = j - rank * p.Hkv;
    b = fp.tseq[min(rank, kFusedSeqs - 1)];
    s = fp.n[b] / chunk;
    k0 = s * chunk;
    k1 = fp.n[b];
  }
  const int ns = (fp.istart[b + 1] - fp.istart[b]) / p.Hkv;
  pslot = fp.istart[b] + h * ns + s;
  ItemDesc d;
  d.b = b;
  d.h = h;
  d.k_begin = k0;
  d.k_end = k1;
  d.t0 = fp.t0[b];
  d.D = fp.dr[b];
  d.N = fp.n[b];
  d.nsplit = ns;
  return d;
}

// ---------------------------------------------------------------------------

// XOR swizzle of the 16-byte chunks of a K row in LDS for verify_attn_main, a
// function of the key's position in the 32-key tile (64 banks of 4 bytes): the
// sixteen key rows one ds_read_b128 reads together ((r/4)*8 + kb*4 + r%4,
// r < 16) land on distinct banks.  Bit 2 of the key (kb) is not used, so the
// rows of the second block sit a constant four rows further.
template <int HD>
__device__ __forceinline__ int key_swz(int k) {
  if constexpr (HD == 128) return (k & 3) | (((k >> 3) & 3) << 2);
  else return ((k >> 1) & 1) | (((k >> 3) & 3) << 1);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The V^T operand of a P V MFMA: eight keys of one head dimension per lane.
// d-major V pages hold them contiguously (one ds_read_b128); key-major pages
// (VKM) need two transposing reads (ds_read_b64_tr_b16: each group of 16
// lanes reads four key rows x 16 dimensions and each lane gets four keys of
// its dimension), the second four key rows further.
template <bool VKM, int ROWB>
__device__ __forceinline__ bf16x8 vt_operand(lds_u8* lds, int off) {
  if constexpr (VKM) {
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off + 4 * ROWB));
    const u32x2 lo = __builtin_bit_cast(u32x2, lo4);
    const u32x2 hi = __builtin_bit_cast(u32x2, hi4);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  } else {
    return *(const bf16x8*)((const __attribute__((address_space(3))) unsigned char*)lds + off);
  }
}


// Reductions over the four lanes {l, l^16, l^32, l^48} that hold one query row.
__device__ __forceinline__ float row_max4(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The max a split-KV partial is stored with: the offset its P values were
// actually computed against.  In the fast pass a row whose first tile of the
// item shows no visible key keeps a reference of -inf and takes its P against
// 0, which happens under a draft-tree mask when a split begins inside the tree
// and the row's own nodes lie in a later tile of the item; such a partial then
// holds l > 0 and must carry 0, not -inf, or the combine weights it by zero.
// A partial with l = 0 keeps -inf so that it cannot raise the merged max.
__device__ __forceinline__ float partial_max(float m, float l) {
  return l > 0.f ? (m == -INFINITY ? 0.f : m) : -INFINITY;
}

template <int HD, int NW, int WPC>
struct Ring {
  static constexpr int kTile = 32;                        // keys per tile (two pages)
  static constexpr int kRowB = HD * 2;                    // bytes per key row
  static constexpr int kCpr = kRowB / 16;                 // 16-byte chunks per row
  static constexpr int kHalf = kTile * kRowB;             // K (or V) bytes per tile
  static constexpr int kStageB = 2 * kHalf;
  static constexpr int kBudget = SDV_RING_BYTES_PER_CU / WPC;
  // even, so that the unrolled tile loop alternates two score buffers statically
  static constexpr int kStages = (kBudget / kStageB < 8 ? kBudget / kStageB : 8) & ~1;
  static constexpr int kLoadsKV = 2 * kHalf / 1024;       // 1 KB DMA instructions per tile (K and V)
  static constexpr int kLPW = kLoadsKV / NW;              // ... per wave
  static constexpr int kKeysPerLoad = 1024 / kRowB;       // key rows one instruction fills
  static_assert(kStages >= 4, "the pipelined tile loop needs four ring stages");
  static_assert(kLoadsKV % NW == 0 && kLPW >= 1, "DMA instructions divide evenly over the waves");
};

// One LDS-DMA instruction of a tile as seen by one lane: it moves 1 KiB (16
// bytes per lane) of one (page, head) block into a ring stage.
//   K: kKeysPerLoad key rows in key order; the lane's 16 bytes are logical
//      chunk (lane % kCpr) ^ swz(key) of its key row.
//   V (d-major pages): 32 d-rows of one V page (16 keys x 2 bytes per d); LDS
//      half h of d-row d holds keys ((h ^ bit 3 of d) * 8)..+7, so that
//      sixteen consecutive d-rows read at one key half land on distinct banks.
//   V (key-major pages, VKM): like K, key rows in key order, with the chunk
//      swizzle vkm_swz of the transposing reads.
struct DmaSlot {
  unsigned src;   // lane's byte offset inside the (page, head) block
  int dst;        // byte offset of the instruction's 1 KiB inside the stage's K (or V) tile
  int page;       // page of the tile (0 or 1)
  int kv;         // 0: K, 1: V
  int key0;       // tile-relative key of the lane's first element
  int rows;       // 1: the lane's 16 bytes are one key's (K, key-major V); 0: eight keys of one dimension
};

// XOR swizzle of the 16-byte chunks of a key-major V row in LDS (period 16
// keys), for the transposing reads of the V^T operand: one read covers key
// rows 16s + {0..3, 8..11} (or + 4) times four chunks (the 32x32x16 kernel), or
// rows 8g + 0..3 of the four 8-key groups times two chunks (16x16x32); both
// touch every bank group exactly twice, and rows k and k + 4 (k & 4 == 0)
// share the swizzle, so the second read of a lane sits 4 rows further.
template <int HD>
__device__ __forceinline__ int vkm_swz(int k) {
  if constexpr (HD == 128) return ((k & 3) << 2) | (((k >> 3) & 1) << 1);
  else return (((k >> 1) & 1) << 2) | (((k >> 3) & 1) << 1);
}

template <int HD, class RG, bool VKM, class SWZ>
__device__ __forceinline__ DmaSlot dma_slot(int j, int lane, SWZ swz) {
  DmaSlot s;
  if (j < RG::kLoadsKV / 2 || VKM) {
    const bool v = j >= RG::kLoadsKV / 2;
    const int row0 = (v ? j - RG::kLoadsKV / 2 : j) * RG::kKeysPerLoad;
    const int key = row0 + lane / RG::kCpr;
    const int lc = (lane % RG::kCpr) ^ (v ? vkm_swz<HD>(key) : swz(key));
    s.src = (unsigned)(((key & 15) * HD + lc * 8) * 2);
    s.dst = row0 * RG::kRowB;
    s.page = row0 / kPage;
    s.kv = v ? 1 : 0;
    s.key0 = key;
    s.rows = 1;
  } else {
    constexpr int kPerPage = HD / 32;             // instructions per V page (32 d-rows of 32 bytes)
    const int jv = j - RG::kLoadsKV / 2;
    const int page = jv / kPerPage;
    const int d = (jv % kPerPage) * 32 + lane / 2;
    const int half = (lane & 1) ^ ((d >> 3) & 1);
    s.src = (unsigned)(d * 32 + half * 16);
    s.dst = page * HD * 32 + (jv % kPerPage) * 1024;
    s.page = page;
    s.kv = 1;
    s.key0 = page * kPage + half * 8;
    s.rows = 0;
  }
  return s;
}

// Zero the elements of this wave's DMA loads of stage `sp` whose keys lie at or
// past `lim` (tile-relative): whole key rows (K, key-major V), single entries
// of the d-major V pages.
template <int LPW, class RG, int S>
__device__ __forceinline__ void zero_keys_past(unsigned char* sp, const DmaSlot (&dma)[LPW], int lane, int lim) {
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    if (dma[i].rows) {
      if (dma[i].key0 >= lim)
        *(u32x4*)(sp + dma[i].kv * S * RG::kHalf + dma[i].dst + lane * 16) = u32x4{0, 0, 0, 0};
    } else if (dma[i].key0 + 7 >= lim) {
      // (compared as q >= lim - key0, so that no key0 + q stays live across the item loop)
      const int nvalid = lim - dma[i].key0;
      unsigned short* e = (unsigned short*)(sp + S * RG::kHalf + dma[i].dst + lane * 16);
      u32x4 x = *(u32x4*)e;
      unsigned short* xs = (unsigned short*)&x;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q >= nvalid) xs[q] = 0;
      *(u32x4*)e = x;
    }
  }
}

// Wait until at most `tiles` tiles' worth (LPW loads each, tiles <= 6) of this
// wave's vector loads are in flight; the count must be an immediate, hence the
// switch.
template <int LPW>
__device__ __forceinline__ void wait_tiles(int tiles) {
  switch (tiles) {
    case 6: wait_vmem<6 * LPW>(); break;
    case 5: wait_vmem<5 * LPW>(); break;
    case 4: wait_vmem<4 * LPW>(); break;
    case 3: wait_vmem<3 * LPW>(); break;
    case 2: wait_vmem<2 * LPW>(); break;
    case 1: wait_vmem<LPW>(); break;
    default: wait_vmem<0>(); break;
  }
}

template <int V>
using ic = std::integral_constant<int, V>;

// f(ic<I>{}) for I = B .. E-1, in order (compile-time indices).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// NRB row blocks of 16 per wave, NW waves, WPC resident workgroups per CU.
template <int HD, int NRB, int NW, int WPC, int OUT_F32, bool TREE, bool VKM>
__global__ __launch_bounds__(64 * NW, WPC) void verify_attn_main(AttnParams p) {
  using RG = Ring<HD, NW, WPC>;
  constexpr int S = RG::kStages;
  constexpr int NKC = HD / 32;   // MFMA k-steps over d for S
  constexpr int NDB = HD / 16;   // 16-wide d blocks of O
  constexpr int LPW = RG::kLPW;
  constexpr int kPageB = kPage * HD * 2;   // bytes of one (page, head) block
  constexpr float kLazy = 8.f;             // safe pass: raise the running max only when it grows by more than 2^8
  constexpr int kPageSlots = kMaxChunk / kPage + 2 * S;
  static_assert(S - 2 <= 6 && (S - 2) * LPW < 64, "wait_tiles range");
  // One LDS object: the K tiles of all ring stages, then the V tiles (so that a
  // lane-constant base plus a 16-bit immediate reaches every stage), then the
  // page ids of the current item.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * RG::kStageB + kPageSlots * 4];
  int* s_pages = (int*)(smem + S * RG::kStageB);
  lds_u8* lds_smem = (lds_u8*)smem;
  const unsigned lds_base = (unsigned)(size_t)lds_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  __shared__ FusedPlan fp;
  if (p.fused) fused_plan(p, fp);
  const int total = __builtin_amdgcn_readfirstlane(min(p.fused ? fp.total : p.plan[1], p.item_cap));
  const int Hq = p.Hkv * p.G;

  // Lane-constant LDS offsets inside a stage (the stage itself is an immediate
  // in the unrolled tile loop).  S^T block kb takes key (r/4)*8 + kb*4 + r%4
  // as its MFMA row r, so that lane group g4 holds the eight consecutive keys
  // g4*8..+7 of the tile: K operand row key(0, l16) (+4 rows for kb = 1),
  // logical chunk c*4 + g4; V^T operand d-row db*16 + l16, keys g4*8..+7.
  const int kkey = (l16 >> 2) * 8 + (l16 & 3);
  int koff[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) koff[c] = kkey * RG::kRowB + (((c * 4 + g4) ^ key_swz<HD>(kkey)) * 16);
  int voffs[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dd = db * 16 + l16;
    if constexpr (VKM) {   // transposing read: key row g4*8 + l16/4 (+4 for the second), dims dd0..+3
      const int key = g4 * 8 + (l16 >> 2);
      const int dd0 = db * 16 + 4 * (l16 & 3);
      voffs[db] = S * RG::kHalf + key * RG::kRowB + (((dd0 >> 3) ^ vkm_swz<HD>(key)) * 16) + (dd0 & 7) * 2;
    } else {
      voffs[db] = S * RG::kHalf + (g4 >> 1) * HD * 32 + dd * 32 + (((g4 & 1) ^ ((dd >> 3) & 1)) * 16);
    }
  }

  // DMA instruction j = wave + NW*i of a tile: K rows for j < kLoadsKV/2, V pages after
  DmaSlot dma[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) dma[i] = dma_slot<HD, RG, VKM>(wave + NW * i, lane, [](int k) { return key_swz<HD>(k); });
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // Items after the first round.  When the plan's list (longest first) holds
  // items shorter than the chunk and more items than workgroups, the next item
  // of this workgroup's class (index = blockIdx % 8 modulo 8) as workgroups
  // finish, from the class's counter; otherwise a fixed stride.
  __shared__ int s_next;
  const int chunk = __builtin_amdgcn_readfirstlane(p.fused ? fp.chunk : p.plan[0]);
  const bool dyn = !p.fused && gridDim.x >= 8 && total > (int)gridDim.x && p.plan[2] < total;
  const int cls = blockIdx.x & 7;
  const int first_dyn = (int)gridDim.x + ((cls - (int)(gridDim.x & 7)) & 7);
  auto next_item = [&](int vi) {
    if (p.fused) {   // snake order over the longest-first list: round r runs forward when r is even
      const int G = (int)gridDim.x, r = vi / G + 1;
      return r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    }
    if (!dyn) return vi + (int)gridDim.x;
    block_sync();
    if (threadIdx.x == 0) s_next = first_dyn + 8 * atomicAdd(p.plan + 8 + cls, 1);
    block_sync_lds();   // (a bare barrier would let a wave read the old index)
    return s_next;
  };
  constexpr int row0 = 0;
  for (int item = blockIdx.x; item < total; item = next_item(item)) {
    int fslot = 0;
    const ItemDesc d = p.fused ? fused_item(p, fp, item, fslot) : p.items[item];
    if (p.fused && threadIdx.x == 0) p.items[item] = d;
    // wave-uniform copies, so that everything derived from them (page bases,
    // tile counts) stays in scalar registers
    const int b = __builtin_amdgcn_readfirstlane(d.b), h = __builtin_amdgcn_readfirstlane(d.h);
    const int k_begin = __builtin_amdgcn_readfirstlane(d.k_begin), k_end = __builtin_amdgcn_readfirstlane(d.k_end);
    const int t0 = __builtin_amdgcn_readfirstlane(d.t0), D = __builtin_amdgcn_readfirstlane(d.D);
    const int N = __builtin_amdgcn_readfirstlane(d.N), nsplit = __builtin_amdgcn_readfirstlane(d.nsplit);
    // (a descriptor outside the inputs is skipped rather than followed)
    if (b < 0 || b >= p.B || h < 0 || h >= p.Hkv || k_begin < 0 || k_end < k_begin ||
        k_end > p.max_pages * kPage || nsplit < 1 || chunk < 64)
      continue;
    const int pslot = p.fused ? __builtin_amdgcn_readfirstlane(fslot)
                              : p.plan[kPlanHeader + b] + h * nsplit + k_begin / chunk;   // natural index: partials
    if (pslot < 0 || pslot >= p.item_cap) continue;
    const int R = p.G * (1 + D);
    const int* bt = p.block_table + (size_t)b * p.max_pages;
    const bool wave_active = row0 + wave * NRB * 16 < R;
    const int ntiles = k_end > k_begin ? (k_end - k_begin + RG::kTile - 1) / RG::kTile : 0;
    const bool ragged_tail = k_begin + ntiles * RG::kTile > k_end;
    const unsigned char* kbase = (const unsigned char*)p.k + (size_t)h * kPageB;
    const unsigned char* vbase = (const unsigned char*)p.v + (size_t)h * kPageB;
    const uint64_t page_stride = (uint64_t)p.Hkv * kPageB;

    // Page ids of a tile's two pages (wave-uniform) -> this wave's DMA loads of
    // the tile into ring stage `st`.
    auto tile_pages = [&](int tile) {
      const u32x2 v = *(const u32x2*)(s_pages + tile * 2);
      return u32x2{(unsigned)__builtin_amdgcn_readfirstlane(v[0]), (unsigned)__builtin_amdgcn_readfirstlane(v[1])};
    };
    auto issue = [&](u32x2 pids, int st) {
      const uint64_t off0 = (uint64_t)pids[0] * page_stride;
      const uint64_t off1 = (uint64_t)pids[1] * page_stride;
      const unsigned sb = lds_base + (unsigned)(st * RG::kHalf);
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        dma16<true>((dma[i].kv ? vbase : kbase) + (dma[i].page ? off1 : off0), dma[i].src,
              sb + (unsigned)(dma[i].kv * S * RG::kHalf + dma[i].dst));
    };
    // zero what this wave loaded into stage st for keys at or past k_end (last
    // tile only); the stores complete here, since the ring barrier that
    // follows is the bare one
    auto zero_tail = [&](int tile, int st) {
      zero_keys_past<LPW, RG, S>(smem + st * RG::kHalf, dma, lane, k_end - (k_begin + tile * RG::kTile));
      wait_lds();
    };

    // Query fragments (B operand of S^T = K Q^T): lane holds row l16, dims g4*8..+7 of each 32-wide step.
    bf16x8 qf[NRB][NKC];
    int pos[NRB];
    unsigned long long tm[NRB];    // draft tree: the nodes row rb sees (bit j: node j of the block)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = row0 + (wave * NRB + rb) * 16 + l16;
      const int i0 = row / p.G;
      const bool valid = row < R && t0 >= 0 && t0 + i0 < p.total_q;
      const int i = valid ? i0 : 0;
      const int g = valid ? row - i * p.G : 0;
      pos[rb] = valid ? N - 1 - D + i : -1;
      tm[rb] = 0ull;
      if constexpr (TREE) tm[rb] = valid ? p.tmask[t0 + i] : 0ull;
      const uint16_t* qp = p.q + ((size_t)(t0 + i) * Hq + (size_t)h * p.G + g) * HD + g4 * 8;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        u32x4 raw = valid ? *(const u32x4*)(qp + c * 32) : u32x4{0, 0, 0, 0};
        qf[rb][c] = __builtin_bit_cast(bf16x8, raw);
      }
    }

    float m_run[NRB];
    float m_off[NRB];              // -m_run, or 0 while m_run is -inf (exp2 argument offset)
    f32x4 l_acc[NRB];              // row sums of P from an MFMA against ones (all four entries equal)
    f32x4 o[NRB][NDB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      m_run[rb] = -INFINITY;
      m_off[rb] = 0.f;
      l_acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Page ids of every page the item's tiles touch (pages past the sequence's
    // last one repeat it, so every DMA reads valid memory), clamped into the
    // pool; then drain every load issued so far so that the ring's vmcnt
    // accounting below only ever sees its own LDS-DMA loads.
    const int page0 = k_begin / kPage;
    const int last_page = (k_end - 1) / kPage;
    for (int j = tid; j < ntiles * (RG::kTile / kPage); j += 64 * NW)
      s_pages[j] = min(max(bt[min(page0 + j, last_page)], 0), p.num_pages - 1);
    wait_vmem<0>();
    block_sync_lds();

    // Scores of tile `tile`: causal (or draft-tree) mask, only for tiles that
    // reach the draft block, and row max.
    f32x4 sc[2][2][NRB];           // scores of tiles of even / odd index
    float mt[NRB];                 // row max of the newest scores (log2 units)
    auto mask_scores = [&](f32x4 (&s)[2][NRB], int tile) {
      const int ts = k_begin + tile * RG::kTile;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if constexpr (TREE) {
          const int nb = ts + g4 * 8 - (N - 1 - D);   // block node of key g4*8 (before the block: < 0, seen)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int node = nb + kb * 4 + e;
              if (!(node < 0 || (node < 64 && ((tm[rb] >> node) & 1ull)))) s[kb][rb][e] = -INFINITY;
            }
        } else {
          const int lim = pos[rb] - ts - g4 * 8;   // key g4*8 + kb*4 + e is visible iff kb*4 + e <= lim
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kb * 4 + e > lim) s[kb][rb][e] = -INFINITY;
        }
      }
    };
    // Sets mt; true if some row's max exceeds its running max by more than `slack`.
    auto row_max = [&](const f32x4 (&s)[2][NRB], float slack) {
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float m = fmaxf(fmaxf(s[0][rb][0], s[0][rb][1]), fmaxf(s[0][rb][2], s[0][rb][3]));
        m = fmaxf(m, fmaxf(fmaxf(s[1][rb][0], s[1][rb][1]), fmaxf(s[1][rb][2], s[1][rb][3])));
        mt[rb] = row_max4(m) * p.scale_log2;
        over |= mt[rb] > m_run[rb] + slack;
      }
      return over;
    };
    // K operand fragments / transposed V fragments of the tile at byte offset
    // `off` of the K (V) region; `off` folds into the instruction's immediate
    // wherever it is a constant.
    auto read_k = [&](int off, bf16x8 (&kf)[2][NKC]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NKC; ++c)
          kf[kb][c] = *(const bf16x8*)(smem + off + kb * 4 * RG::kRowB + koff[c]);
    };
    auto read_v = [&](int off, bf16x8 (&vf)[NDB]) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) vf[db] = vt_operand<VKM, RG::kRowB>(lds_smem, off + voffs[db]);
    };
    // the 2*NRB accumulation chains advance together (k-step outermost), so
    // consecutive MFMAs never depend on each other
    auto mfma_scores = [&](const bf16x8 (&kf)[2][NKC], f32x4 (&s)[2][NRB]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][c], qf[rb][c], s[kb][rb], 0, 0, 0);
    };
    // P = 2^(S * scale * log2 e - m) in bf16, keys in the order of the S^T accumulators
    auto probs = [&](const f32x4 (&s)[2][NRB], bf16x8 (&pf)[NRB]) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pf[rb][kb * 4 + e] = (__bf16)fast_exp2(fmaf(s[kb][rb][e], p.scale_log2, m_off[rb]));
    };
    // O^T += V^T P^T; l += 1^T P^T
    auto accumulate = [&](const bf16x8 (&vf)[NDB], const bf16x8 (&pf)[NRB]) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf[rb], o[rb][db], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        l_acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[rb], l_acc[rb], 0, 0, 0);
    };

    // ---- Fast pass.  Each row's reference max is fixed by the item's first
    // tile and never moves, and later tiles take no row max at all: a score
    // that rises far above the reference shows in the row sum l (it holds every
    // P), and an item whose l ends above kOverflow (or is not finite) is
    // recomputed by the safe pass below with a running max.  Below that bound
    // o and l are far from fp32 overflow.
    constexpr float kOverflow = 0x1p64f;   // row sums above this redo the item
    // Tiles 0..plain-1 run as pipelined steps: each has a next tile that needs
    // no causal mask.  The first `steady` of them (a multiple of S) run in the
    // unrolled loop with no per-step guards.
    const int plain = max(0, min(ntiles - 1, (N - D - k_begin) / RG::kTile - 1));
    const int steady = plain - plain % S;

    // Tile t (ring stage t % S), pipelined: P of tile t on the vector ALUs
    // while the matrix cores compute the scores of tile t+1, then P V of tile t
    // on the matrix cores while the vector ALUs take the row max of tile t+1.
    auto body = [&](auto uc) {
      constexpr int u = decltype(uc)::value;
      bf16x8 kf[2][NKC];
      read_k(((u + 1) % S) * RG::kHalf, kf);
      bf16x8 vf[NDB];
      read_v(u * RG::kHalf, vf);
      bf16x8 pf[NRB];
      probs(sc[u & 1], pf);
      mfma_scores(kf, sc[(u + 1) & 1]);
      accumulate(vf, pf);
      // interleave: LDS reads first, then one MFMA per few VALU ops
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKC, 0);
#pragma unroll
      for (int i = 0; i < 2 * NRB * NKC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        if (i < NDB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NRB * (NDB + 1), 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8 * NRB, 0);   // the new scores leave the accumulators last
    };

    // The whole tile loop in two copies, for waves with and without query
    // rows in this item, so that no branch inside it merges accumulators.
    auto fast_pass = [&](auto activec) {
      constexpr bool ACTIVE = decltype(activec)::value;
#pragma unroll
      for (int t = 0; t < S - 1; ++t)
        if (t < ntiles) issue(tile_pages(t), t);
      u32x2 pids_next = {0u, 0u};    // page ids of the next tile to issue (tile S-1 first)
      if (S - 1 < ntiles) pids_next = tile_pages(S - 1);
      if (ntiles == 0) return;
      wait_tiles<LPW>(min(S - 2, ntiles - 1));
      if (ntiles == 1 && ragged_tail) zero_tail(0, 0);
      block_sync();
      if constexpr (ACTIVE) {
        bf16x8 kf[2][NKC];
        read_k(0, kf);
        mfma_scores(kf, sc[0]);
        if (k_begin + RG::kTile > N - D) mask_scores(sc[0], 0);
        row_max(sc[0], 0.f);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          m_run[rb] = mt[rb];
          m_off[rb] = mt[rb] == -INFINITY ? 0.f : -mt[rb];
        }
      }
      // wait for tile t+1, barrier, refill the stage tile t-1 used with tile t+S-1
      auto advance = [&](int t, int st_issue) {
        wait_tiles<LPW>(min(S - 3, ntiles - 2 - t));
        if (t + 1 == ntiles - 1 && ragged_tail) zero_tail(t + 1, (t + 1) % S);
        block_sync();
        if (t + S - 1 < ntiles) {
          issue(pids_next, st_issue);
          if (t + S < ntiles) pids_next = tile_pages(t + S);
        }
      };
      for (int tb = 0; tb < steady; tb += S) {
        auto step = [&](auto uc) {
          constexpr int u = decltype(uc)::value;
          advance(tb + u, (u + S - 1) % S);
          if constexpr (ACTIVE) body(uc);
        };
        step(ic<0>{});
        step(ic<1>{});
        step(ic<2>{});
        step(ic<3>{});
        if constexpr (S > 4) step(ic<4>{});
        if constexpr (S > 5) step(ic<5>{});
        if constexpr (S > 6) step(ic<6>{});
        if constexpr (S > 7) step(ic<7>{});
      }
      // the plain tiles past the last whole block (fewer than S): the same
      // pipelined steps behind one uniform guard each.  Their ring stages stay
      // static (steady is a multiple of S); afterwards the next tile's scores
      // are moved to sc[0], where the tail takes them.
      {
        const int extra = plain - steady;
        auto step = [&](auto uc) {
          constexpr int u = decltype(uc)::value;
          if constexpr (u < S - 1) {
            if (u < extra) {
              advance(steady + u, (u + S - 1) % S);
              if constexpr (ACTIVE) body(uc);
            }
          }
        };
        step(ic<0>{});
        step(ic<1>{});
        step(ic<2>{});
        step(ic<3>{});
        step(ic<4>{});
        step(ic<5>{});
        step(ic<6>{});
        if constexpr (ACTIVE) {
          if (extra & 1) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int rb = 0; rb < NRB; ++rb) sc[0][kb][rb] = sc[1][kb][rb];
          }
        }
      }
      // tail: the masked tiles and the last one, one at a time with run-time ring stages
      for (int t = plain; t < ntiles; ++t) {
        const bool has_next = t + 1 < ntiles;
        if (has_next) {
          advance(t, (t + S - 1) % S);
        } else {
          block_sync();
        }
        if constexpr (ACTIVE) {
          bf16x8 pf[NRB];
          probs(sc[0], pf);
          bf16x8 vf[NDB];
          read_v((t % S) * RG::kHalf, vf);
          accumulate(vf, pf);
          if (has_next) {
            bf16x8 kf[2][NKC];
            read_k(((t + 1) % S) * RG::kHalf, kf);
            mfma_scores(kf, sc[0]);
            if (k_begin + (t + 2) * RG::kTile > N - D) mask_scores(sc[0], t + 1);
          }
        }
      }
    };
    if (wave_active) fast_pass(std::true_type{});
    else fast_pass(std::false_type{});
    // every load of the fast pass has landed (the last tile waited for vmcnt 0)
    bool over = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) over |= !(l_acc[rb][0] <= kOverflow);
    over &= wave_active;

    // ---- Safe pass (only if some row's max outgrew the fast pass): the same
    // tiles again, one at a time, with a running max raised lazily (when it
    // grows by more than 2^kLazy) and the accumulators rescaled.
    if (__syncthreads_or(over ? 1 : 0)) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        m_run[rb] = -INFINITY;
        m_off[rb] = 0.f;
        l_acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int t = 0; t < S - 1; ++t)
        if (t < ntiles) issue(tile_pages(t), t);
      for (int t = 0; t < ntiles; ++t) {
        wait_tiles<LPW>(min(S - 2, ntiles - 1 - t));
        if (t == ntiles - 1 && ragged_tail) zero_tail(t, t % S);
        block_sync();
        if (t + S - 1 < ntiles) issue(tile_pages(t + S - 1), (t + S - 1) % S);
        if (wave_active) {
          const int off = (t % S) * RG::kHalf;
          bf16x8 kf[2][NKC];
          read_k(off, kf);
          mfma_scores(kf, sc[0]);
          if (k_begin + (t + 1) * RG::kTile > N - D) mask_scores(sc[0], t);
          if (__any(row_max(sc[0], kLazy))) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
              if (mt[rb] > m_run[rb] + kLazy) {
                const float alpha = fast_exp2(m_run[rb] - mt[rb]);
                m_run[rb] = mt[rb];
                m_off[rb] = -mt[rb];
                l_acc[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[rb][db] *= alpha;
              }
            }
          }
          bf16x8 pf[NRB];
          probs(sc[0], pf);
          bf16x8 vf[NDB];
          read_v(off, vf);
          accumulate(vf, pf);
        }
      }
    }
    // every wave is done with the ring before the next item's loads land in it
    block_sync();

    if (wave_active) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float lt = l_acc[rb][0];
        const int row = row0 + (wave * NRB + rb) * 16 + l16;
        if (row >= R || t0 < 0 || t0 + row / p.G >= p.total_q) continue;
        if (nsplit == 1) {
          const int i = row / p.G;
          const int g = row - i * p.G;
          const float inv = lt > 0.f ? 1.f / lt : 0.f;
          const size_t obase = ((size_t)(t0 + i) * Hq + (size_t)h * p.G + g) * HD + g4 * 4;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const f32x4 v = o[rb][db] * inv;
            if (OUT_F32) {
              *(f32x4*)((float*)p.out + obase + db * 16) = v;
            } else {
              const bf16x4 t = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
              *(u32x2*)((uint16_t*)p.out + obase + db * 16) = __builtin_bit_cast(u32x2, t);
            }
          }
        } else {
          float* slab = p.part_o + ((size_t)pslot * p.rpad + row) * HD + g4 * 4;
#pragma unroll
          for (int db = 0; db < NDB; ++db) *(f32x4*)(slab + db * 16) = o[rb][db];
          if (g4 == 0) {
            float* ml = p.part_ml + ((size_t)pslot * p.rpad + row) * 2;
            ml[0] = partial_max(m_run[rb], lt);
            ml[1] = lt;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Verify attention with 32x32x16 MFMAs for blocks of more than 64 query rows:
// a workgroup of 8 waves, two per SIMD, in two sets of four (32 rows per
// wave), both fed from one LDS-DMA ring.  Up to 128 rows (MODE 0), set 0
// takes the even tiles of the item and set 1 the odd ones over the same 128
// rows, and the two partial results are merged through LDS at the end of the
// item.  Up to 256 rows (MODE 1), set s takes rows 128s .. 128s+127 over every
// tile, so the item's pages are streamed once for all its rows.  From 129 to
// 192 rows (MODE 2) set 0 takes rows 0..127 over every tile and set 1 splits
// the tiles of the remaining one or two row blocks; from 129 to 144 rows
// (MODE 3) the rows past 128 form one 16-row block of 16x16x32 MFMAs, whose
// tiles two waves of set 1 split.  Two waves per SIMD hide
// each other's LDS, barrier and MFMA-dependency latencies.  Operands:
//   * S^T = K Q^T per 32-key tile: A = K (lane: key row l%32, dims
//     c*16 + (l/32)*8..+7), B = Q^T (lane: query row l%32, same dims), so each
//     lane holds one query row and keys (e/4)*8 + (l/32)*4 + e%4, e < 16.
//   * O^T += V^T P^T per 16-key step ks: A = V^T read transposed, keys in the
//     accumulator's order (ks*16 + (l/32)*4 + 0..3, then +8); B = P^T, which is
//     entries 8ks..8ks+7 of the score accumulator converted to bf16.
// Reference maxima, the overflow check and the safe pass follow
// verify_attn_main.

// XOR swizzle of the 16-byte chunks of a K or V row in LDS for this kernel, a
// function of the key's position mod 16 (64 banks of 4 bytes): sixteen
// consecutive key rows read at one logical chunk (the K operand) land on
// distinct banks, and so do four consecutive key rows times an aligned run of
// four chunks (one transposed V read of 32 lanes).
template <int HD>
__device__ __forceinline__ int wide_swz(int k) {
  if constexpr (HD == 128) return ((k & 3) << 2) | ((k >> 2) & 3);
  else return (((k >> 1) & 1) << 2) | ((k >> 2) & 3);
}

// MODE 0 (up to 128 rows): the two wave sets split the tiles of every step
// over the same four 32-row blocks.  MODE 1 (up to 256 rows): each wave takes
// one of eight row blocks over both tiles of every step.  MODE 2 (129 to 192
// rows): waves 0-3 take row blocks 0-3 over both tiles, and waves 4-7 share
// blocks 4 and 5 two to a block, one tile of every step each, so that no SIMD
// (it hosts waves s and s+4) carries more than three of the step's 32-row
// tile products where the row split would give one SIMD four.  MODE 3 (129 to
// 144 rows): waves 0-3 as in MODE 2; waves 4 and 5 take rows 128..143 as a
// 16-row block, one tile of every step each, so the rows past 128 cost a
// quarter of a 32-row tile product per tile instead of a half; waves 6 and 7
// only load.
//
// The 16-row block (16x16x32 MFMAs, as verify_attn_main): S^T block kb takes
// key (r/4)*8 + kb*4 + r%4 as its MFMA row r, so lane group g = l/16 holds the
// eight consecutive keys 8g..8g+7 of the tile (entries kb*4 + e) for query row
// 128 + l%16, which is the B operand of O^T += V^T P^T over the whole tile.
// Its registers are those of the 32-row path: Q in qf[0 .. HD/32), the K
// offsets of block kb in koff[kb*HD/32 ..], the scores in sc[0..7] and the
// output block db (d = 16db + 4g + 0..3) in entries 4(db%4) .. of o[db/4].
template <int HD, int OUT_F32, int MODE, bool TREE, bool VKM>
__global__ __launch_bounds__(512, 1) void verify_attn_wide(AttnParams p) {
  constexpr int NW = 8;
  using RG = Ring<HD, NW, 1>;
  constexpr int S = RG::kStages;
  constexpr int NKS = HD / 16;   // 16-wide d steps of S^T
  constexpr int NMB = HD / 32;   // 32-wide d blocks of O^T
  constexpr int LPW = RG::kLPW;
  constexpr int kPageB = kPage * HD * 2;
  constexpr float kLazy = 8.f;   // safe pass: raise the running max only when it grows by more than 2^8
  constexpr float kOverflow = 0x1p64f;   // row sums above this redo the item
  constexpr int kPageSlots = kMaxChunk / kPage + 2 * S;
  constexpr int kMergeF = 16 * NMB + 2;        // floats per lane handed from set 1 to set 0
  static_assert(S % 2 == 0 && S >= 6 && (S - 4) <= 6 && (S - 4) * LPW < 64, "ring depth");
  static_assert(4 * kMergeF * 64 * 4 <= S * RG::kStageB, "merge buffer fits in the ring");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * RG::kStageB + kPageSlots * 4];
  int* s_pages = (int*)(smem + S * RG::kStageB);
  lds_u8* lds_smem = (lds_u8*)smem;
  const unsigned lds_base = (unsigned)(size_t)lds_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int set = wave >> 2, w4 = wave & 3;
  const int r32 = lane & 31, hh = lane >> 5;
  // This wave's role: PAIR waves take both tiles of a step, the others the
  // tile of parity `par`; its 32-row block; whether it hands its partial to
  // a partner (same block, other parity) through LDS, and where.
  const bool pair = MODE == 1 || (MODE >= 2 && set == 0);
  const bool narrow = MODE == 3 && set == 1;     // the 16-row block (waves 4 and 5; 6 and 7 idle)
  const int par = MODE == 0 ? set : (MODE >= 2 && set == 1) ? (w4 & 1) : 0;
  const int rblock = MODE == 0 ? w4 : MODE == 1 ? wave : set == 0 ? w4 : MODE == 3 ? 4 + 2 * (w4 >> 1) : 4 + (w4 >> 1);
  const bool giver = !pair && par == 1;          // hands (O, l, m) to the block's parity-0 wave
  const int xslot = MODE == 0 ? w4 : (w4 >> 1);  // LDS hand-off slot of the block
  __shared__ FusedPlan fp;
  if (p.fused) fused_plan(p, fp);
  const int total = __builtin_amdgcn_readfirstlane(min(p.fused ? fp.total : p.plan[1], p.item_cap));
  const int Hq = p.Hkv * p.G;

  // Lane-constant LDS offsets, including (single-tile waves) the stage parity:
  // in step k such a wave reads tile 2k + par, whose stage is (2k + par) % S.
  // PAIR waves read both tiles of the step.
  // S^T takes key pi(r) = (r/16)*16 + ((r/4)%2)*8 + ((r/8)%2)*4 + r%4 as its MFMA
  // row r, so that score entry e of a lane holds key (e/8)*16 + 8hh + e%8 and
  // each 16-key step of P V reads eight consecutive keys per lane.
  const int kkey = (r32 >> 4) * 16 + ((r32 >> 2) & 1) * 8 + ((r32 >> 3) & 1) * 4 + (r32 & 3);
  int koff[NKS];                 // K operand: key row kkey, logical chunk 2c + hh
#pragma unroll
  for (int c = 0; c < NKS; ++c)
    koff[c] = par * RG::kHalf + kkey * RG::kRowB + (((c * 2 + hh) ^ wide_swz<HD>(kkey)) * 16);
  int voffs[NMB];                // V^T operand: d-row mb*32 + r32, keys ks*16 + 8hh..+7 (page ks)
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int dd = mb * 32 + r32;
    if constexpr (VKM) {   // transposing read: key row 8hh + j16/4 (+4 for the second), dims dd0..+3
      const int j16 = lane & 15;
      const int key = 8 * hh + (j16 >> 2);
      const int dd0 = mb * 32 + 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
      voffs[mb] = par * RG::kHalf + S * RG::kHalf + key * RG::kRowB + (((dd0 >> 3) ^ vkm_swz<HD>(key)) * 16) +
                  (dd0 & 7) * 2;
    } else {
      voffs[mb] = par * RG::kHalf + S * RG::kHalf + dd * 32 + ((hh ^ ((dd >> 3) & 1)) * 16);
    }
  }
  // The 16-row block's operands (lane l16 = l % 16, group g4 = l / 16).  K of
  // S^T block kb: key row (l16/4)*8 + kb*4 + l16%4, logical chunk 4c + g4, in
  // koff[kb * NKC16 + c].  V^T block db: d-rows 16db + l16, keys 8g4..+7, at
  // voffs[0] + 512 db (d-major pages) or, key-major, at voffs[0] + 32 (db ^
  // voffs[1]) (key row 8g4 + l16/4, dims 16db + 4(l16 % 4)..+3, whose chunk
  // pair 2db.. the row's swizzle permutes).
  constexpr int NKC16 = HD / 32;   // 32-wide d steps of the 16-row S^T
  constexpr int NDB16 = HD / 16;   // 16-row d blocks of O^T
  if constexpr (MODE == 3) {
    if (narrow) {
      const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = (l16 >> 2) * 8 + kb * 4 + (l16 & 3);
#pragma unroll
        for (int c = 0; c < NKC16; ++c)
          koff[kb * NKC16 + c] = par * RG::kHalf + key * RG::kRowB + (((c * 4 + g4) ^ wide_swz<HD>(key)) * 16);
      }
      if constexpr (VKM) {
        const int key = 8 * g4 + (l16 >> 2);
        const int sw = vkm_swz<HD>(key);   // (bit 0 clear: the chunk pair of a d block stays a pair)
        voffs[0] = par * RG::kHalf + S * RG::kHalf + key * RG::kRowB + ((((l16 & 3) >> 1) ^ (sw & 1)) * 16) +
                   ((4 * (l16 & 3)) & 7) * 2;
        voffs[1] = sw >> 1;
      } else {
        voffs[0] = par * RG::kHalf + S * RG::kHalf + (g4 >> 1) * HD * 32 + l16 * 32 +
                   (((g4 & 1) ^ ((l16 >> 3) & 1)) * 16);
      }
    }
  }
  DmaSlot dma[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i)
    dma[i] = dma_slot<HD, RG, VKM>(wave + NW * i, lane, [](int k) { return wide_swz<HD>(k & 15); });

  // Items after the first round.  When the plan's list (longest first) holds
  // items shorter than the chunk and more items than workgroups, the next item
  // of this workgroup's class (index = blockIdx % 8 modulo 8) as workgroups
  // finish, from the class's counter; otherwise a fixed stride.
  __shared__ int s_votes[NW];    // MODE 3: per-wave votes of the safe-pass test
  __shared__ int s_next;
  const int chunk = __builtin_amdgcn_readfirstlane(p.fused ? fp.chunk : p.plan[0]);
  const bool dyn = !p.fused && gridDim.x >= 8 && total > (int)gridDim.x && p.plan[2] < total;
  const int cls = blockIdx.x & 7;
  const int first_dyn = (int)gridDim.x + ((cls - (int)(gridDim.x & 7)) & 7);
  auto next_item = [&](int vi) {
    if (p.fused) {   // snake order over the longest-first list: round r runs forward when r is even
      const int G = (int)gridDim.x, r = vi / G + 1;
      return r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    }
    if (!dyn) return vi + (int)gridDim.x;
    block_sync();
    if (threadIdx.x == 0) s_next = first_dyn + 8 * atomicAdd(p.plan + 8 + cls, 1);
    block_sync_lds();   // (a bare barrier would let a wave read the old index)
    return s_next;
  };
  for (int item = blockIdx.x; item < total; item = next_item(item)) {
    int fslot = 0;
    const ItemDesc d = p.fused ? fused_item(p, fp, item, fslot) : p.items[item];
    if (p.fused && threadIdx.x == 0) p.items[item] = d;
    const int b = __builtin_amdgcn_readfirstlane(d.b), h = __builtin_amdgcn_readfirstlane(d.h);
    const int k_begin = __builtin_amdgcn_readfirstlane(d.k_begin), k_end = __builtin_amdgcn_readfirstlane(d.k_end);
    const int t0 = __builtin_amdgcn_readfirstlane(d.t0), D = __builtin_amdgcn_readfirstlane(d.D);
    const int N = __builtin_amdgcn_readfirstlane(d.N), nsplit = __builtin_amdgcn_readfirstlane(d.nsplit);
    // (a descriptor outside the inputs is skipped rather than followed)
    if (b < 0 || b >= p.B || h < 0 || h >= p.Hkv || k_begin < 0 || k_end < k_begin ||
        k_end > p.max_pages * kPage || nsplit < 1 || chunk < 64)
      continue;
    const int pslot = p.fused ? __builtin_amdgcn_readfirstlane(fslot)
                              : p.plan[kPlanHeader + b] + h * nsplit + k_begin / chunk;   // natural index: partials
    if (pslot < 0 || pslot >= p.item_cap) continue;
    const int R = p.G * (1 + D);
    const int* bt = p.block_table + (size_t)b * p.max_pages;
    const bool wave_active = rblock * 32 < R;
    const int ntiles = k_end > k_begin ? (k_end - k_begin + RG::kTile - 1) / RG::kTile : 0;
    const int nsteps = (ntiles + 1) / 2;
    const bool ragged_tail = k_begin + ntiles * RG::kTile > k_end;
    const unsigned char* kbase = (const unsigned char*)p.k + (size_t)h * kPageB;
    const unsigned char* vbase = (const unsigned char*)p.v + (size_t)h * kPageB;
    const uint64_t page_stride = (uint64_t)p.Hkv * kPageB;

    auto tile_pages = [&](int tile) {
      const u32x2 v = *(const u32x2*)(s_pages + tile * 2);
      return u32x2{(unsigned)__builtin_amdgcn_readfirstlane(v[0]), (unsigned)__builtin_amdgcn_readfirstlane(v[1])};
    };
    auto issue = [&](u32x2 pids, int st) {
      const uint64_t off0 = (uint64_t)pids[0] * page_stride;
      const uint64_t off1 = (uint64_t)pids[1] * page_stride;
      const unsigned sb = lds_base + (unsigned)(st * RG::kHalf);
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        dma16<true>((dma[i].kv ? vbase : kbase) + (dma[i].page ? off1 : off0), dma[i].src,
              sb + (unsigned)(dma[i].kv * S * RG::kHalf + dma[i].dst));
    };
    // (as in verify_attn_main: the zeroing stores complete before the bare ring barrier)
    auto zero_tail = [&](int tile) {
      zero_keys_past<LPW, RG, S>(smem + (tile % S) * RG::kHalf, dma, lane, k_end - (k_begin + tile * RG::kTile));
      wait_lds();
    };

    // MODE 3: the lane index, opaque to the compiler once per item, so that
    // the lane terms of the Q and output addresses are formed here, not
    // hoisted out of the item loop as 64-bit pointers held (or spilled) across
    // it.
    int lane_i = lane;
    if constexpr (MODE == 3) asm volatile("" : "+v"(lane_i));
    // Query fragments (B operand of S^T): lane holds row r32, dims c*16 + hh*8..+7
    // (the 16-row block: row 128 + l16, dims c*32 + g4*8..+7 for c < NKC16).
    const int row = narrow ? 128 + (lane & 15) : rblock * 32 + r32;
    const int i0 = row / p.G;
    const bool valid = row < R && t0 >= 0 && t0 + i0 < p.total_q;
    const int qi = valid ? i0 : 0;
    const int qg = valid ? row - qi * p.G : 0;
    const int pos = valid ? N - 1 - D + qi : -1;
    unsigned long long tm = 0ull;   // draft tree: nodes this row sees
    if constexpr (TREE) tm = valid ? p.tmask[t0 + qi] : 0ull;
    bf16x8 qf[NKS];
    if (MODE == 3 && narrow) {
      const uint16_t* qp = p.q + ((size_t)(t0 + qi) * Hq + (size_t)h * p.G + qg) * HD + (lane_i >> 4) * 8;
#pragma unroll
      for (int c = 0; c < NKS; ++c) {
        u32x4 raw = valid && c < NKC16 ? *(const u32x4*)(qp + c * 32) : u32x4{0, 0, 0, 0};
        qf[c] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      const uint16_t* qp = p.q + ((size_t)(t0 + qi) * Hq + (size_t)h * p.G + qg) * HD + (lane_i >> 5) * 8;
#pragma unroll
      for (int c = 0; c < NKS; ++c) {
        u32x4 raw = valid ? *(const u32x4*)(qp + c * 16) : u32x4{0, 0, 0, 0};
        qf[c] = __builtin_bit_cast(bf16x8, raw);
      }
    }
    float m_run = -INFINITY;
    float m_off = 0.f;
    f32x16 mneg;                   // fast pass: -(reference max)/scale in every entry, the score chains' initial value
    float l_run;                   // this lane's share of its row sum (its 16 of each tile's 32 keys);
                                   // the row's sum adds the partner lane l ^ 32
    f32x16 o[NMB];
    auto clear = [&]() {
      m_run = -INFINITY;
      m_off = 0.f;
      l_run = 0.f;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mb][e] = 0.f;
    };
    clear();

    const int page0 = k_begin / kPage;
    const int last_page = (k_end - 1) / kPage;
    for (int j = tid; j < ntiles * (RG::kTile / kPage); j += 64 * NW)
      s_pages[j] = min(max(bt[min(page0 + j, last_page)], 0), p.num_pages - 1);
    wait_vmem<0>();
    block_sync_lds();

    f32x16 sc;
    float mt = -INFINITY;
    auto mask_scores = [&](int tile) {
      if (MODE == 3 && narrow) {   // entry e: key 8g4 + e
        const int g4 = lane >> 4;
        if constexpr (TREE) {
          const int nb = k_begin + tile * RG::kTile + 8 * g4 - (N - 1 - D);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int node = nb + e;
            if (!(node < 0 || (node < 64 && ((tm >> node) & 1ull)))) sc[e] = -INFINITY;
          }
        } else {
          const int lim = pos - (k_begin + tile * RG::kTile) - 8 * g4;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e > lim) sc[e] = -INFINITY;
        }
        return;
      }
      if constexpr (TREE) {
        const int nb = k_begin + tile * RG::kTile + 8 * hh - (N - 1 - D);   // block node of entry 0
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int node = nb + (e >> 3) * 16 + (e & 7);
          if (!(node < 0 || (node < 64 && ((tm >> node) & 1ull)))) sc[e] = -INFINITY;
        }
      } else {
        const int lim = pos - (k_begin + tile * RG::kTile) - 8 * hh;   // key (e/8)*16 + 8hh + e%8 is visible iff (e/8)*16 + e%8 <= lim
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((e >> 3) * 16 + (e & 7) > lim) sc[e] = -INFINITY;
      }
    };
    auto row_max = [&](float slack) {
      float m = sc[0];
      if (MODE == 3 && narrow) {
#pragma unroll
        for (int e = 1; e < 8; ++e) m = fmaxf(m, sc[e]);
        mt = row_max4(m) * p.scale_log2;
        return mt > m_run + slack;
      }
#pragma unroll
      for (int e = 1; e < 16; ++e) m = fmaxf(m, sc[e]);
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      mt = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])) * p.scale_log2;   // (scale > 0)
      return mt > m_run + slack;
    };
    // S^T = K Q^T of the set's tile at stage offset `off`, unscaled (Q stays the
    // exact bf16 input; the fp32 scale scale*log2(e) is applied to each fp32
    // score before the exp).  PRE (fast pass after the first step): one chain
    // that starts from mneg = -(reference max)/scale, so the MFMAs leave the
    // scores less the reference max and P = 2^(scale * s) takes one multiply.
    // Otherwise two chains from zero, whose sum takes one add per score.  (With
    // two waves per SIMD the other wave's MFMAs fill the single chain's
    // dependency stalls: measured, one chain with no adds beats two chains by
    // 1-3%.)
    // The 16-row block's S^T: two 16-key blocks, chains from zero (PRE: from
    // the reference max, as below).
    auto narrow_scores = [&](int off, auto prec) {
      f32x4 s0 = decltype(prec)::value ? f32x4{mneg[0], mneg[1], mneg[2], mneg[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 s1 = s0;
#pragma unroll
      for (int c = 0; c < NKC16; ++c) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(smem + off + koff[c]), qf[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(smem + off + koff[NKC16 + c]), qf[c], s1, 0, 0,
                                                     0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) { sc[e] = s0[e]; sc[4 + e] = s1[e]; }
    };
    auto scores = [&](int off, auto prec) {
      if (MODE == 3 && narrow) return narrow_scores(off, prec);
      if constexpr (decltype(prec)::value) {
        f32x16 s0 = mneg;
#pragma unroll
        for (int c = 0; c < NKS; ++c)
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(smem + off + koff[c]), qf[c], s0, 0, 0, 0);
        sc = s0;
        return;
      }
      f32x16 s0, s1;
#pragma unroll
      for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
#pragma unroll
      for (int c = 0; c < NKS; c += 2) {
        const bf16x8 k0 = *(const bf16x8*)(smem + off + koff[c]);
        const bf16x8 k1 = *(const bf16x8*)(smem + off + koff[c + 1]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[c + 1], s1, 0, 0, 0);
      }
      sc = s0 + s1;
    };
    // P = 2^(scale * score - reference max) in bf16 (PRE: the scores already hold the difference, unscaled)
    auto p_of = [&](float x, auto prec) {
      if constexpr (decltype(prec)::value) return (__bf16)fast_exp2(x * p.scale_log2);
      else return (__bf16)fast_exp2(fmaf(x, p.scale_log2, m_off));
    };
    // P from the scores, then O^T += V^T P^T at stage offset `off`, and the
    // lane's share of l from the same bf16 P (dot products with (1, 1))
    // The 16-row block's P (keys 8g4..+7), O^T block db += V^T P^T, and l.
    auto narrow_accumulate = [&](int off, auto prec) {
      bf16x8 pn;
#pragma unroll
      for (int e = 0; e < 8; ++e) pn[e] = p_of(sc[e], prec);
#pragma unroll
      for (int db = 0; db < NDB16; ++db) {
        const int vo = VKM ? voffs[0] + 32 * (db ^ voffs[1]) : voffs[0] + 512 * db;
        const bf16x8 vf = vt_operand<VKM, RG::kRowB>(lds_smem, off + vo);
        f32x4 acc = {o[db / 4][4 * (db % 4)], o[db / 4][4 * (db % 4) + 1], o[db / 4][4 * (db % 4) + 2],
                     o[db / 4][4 * (db % 4) + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pn, acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db / 4][4 * (db % 4) + e] = acc[e];
      }
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pn[2 * q], pn[2 * q + 1]}, one2, l_run, false);
    };
    auto accumulate = [&](int off, auto prec) {
      if (MODE == 3 && narrow) return narrow_accumulate(off, prec);
      bf16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[ks][e] = p_of(sc[ks * 8 + e], prec);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const bf16x8 vf = vt_operand<VKM, RG::kRowB>(lds_smem, off + ks * HD * 32 + voffs[mb]);
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[mb], 0, 0, 0);
        }
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][2 * q], pf[ks][2 * q + 1]}, one2, l_run, false);
      asm volatile("" ::"v"(l_run));   // keep the sums here: sunk past later tiles they hold P live
    };
    // Row-split steady step over the tiles A (at `off0`) and B (at `off1`) as
    // one fixed sequence of 2 NKS + 4 NMB slots, one MFMA each: S_A; S_B with
    // P_A; P V of A with P_B; P V of B.  In a slot of the second and third
    // phases the wave also issues one share of the other tile's exp / convert /
    // row-sum work, which the SIMD runs while the MFMA occupies the matrix core,
    // and each MFMA's LDS operand is read kAhead slots before it.  Scheduling
    // fences between slots keep that order (left to itself the compiler runs
    // the MFMAs back to back and the vector work after them).
    auto rs_pair = [&](int off0, int off1) {
      constexpr int kSlots = 2 * NKS + 4 * NMB;
      constexpr int kAhead = SDV_RS_AHEAD;
      auto operand = [&](auto jc) -> bf16x8 {            // the LDS operand of slot j
        constexpr int j = decltype(jc)::value;
        if constexpr (j < NKS) return *(const bf16x8*)(smem + off0 + koff[j]);
        else if constexpr (j < 2 * NKS) return *(const bf16x8*)(smem + off1 + koff[j - NKS]);
        else if constexpr (j < 2 * NKS + 2 * NMB)
          return vt_operand<VKM, RG::kRowB>(lds_smem, off0 + ((j - 2 * NKS) / NMB) * HD * 32 + voffs[(j - 2 * NKS) % NMB]);
        else
          return vt_operand<VKM, RG::kRowB>(lds_smem, off1 + ((j - 2 * NKS - 2 * NMB) / NMB) * HD * 32 +
                                                      voffs[(j - 2 * NKS - 2 * NMB) % NMB]);
      };
      // share q of nq of a tile's P work: its 16/nq scores -> exp2 -> bf16 -> row sum
      auto p_share = [&](const f32x16& sv, bf16x8 (&pf)[2], auto qc, auto nqc) {
        constexpr int q = decltype(qc)::value, nq = decltype(nqc)::value;
        constexpr int w = 16 / nq;
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int e = q * w; e < (q + 1) * w; e += 2) {
          pf[e / 8][e % 8] = (__bf16)fast_exp2(sv[e] * p.scale_log2);
          pf[e / 8][e % 8 + 1] = (__bf16)fast_exp2(sv[e + 1] * p.scale_log2);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[e / 8][e % 8], pf[e / 8][e % 8 + 1]}, one2, l_run, false);
        }
        asm volatile("" ::"v"(l_run));   // the sums stay in their slot (sunk, they would hold P live)
      };
      f32x16 sa = mneg, sb = mneg;
      bf16x8 pa[2], pb[2];
      bf16x8 f[kSlots];
      static_for<0, kAhead>([&](auto jc) { f[decltype(jc)::value] = operand(jc); });
      static_for<0, kSlots>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j + kAhead < kSlots) f[j + kAhead] = operand(ic<j + kAhead>{});
        if constexpr (j < NKS) {
          sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j], qf[j], sa, 0, 0, 0);
        } else if constexpr (j < 2 * NKS) {
          sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j], qf[j - NKS], sb, 0, 0, 0);
          p_share(sa, pa, ic<j - NKS>{}, ic<NKS>{});
        } else if constexpr (j < 2 * NKS + 2 * NMB) {
          constexpr int t = j - 2 * NKS;
          o[t % NMB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j], pa[t / NMB], o[t % NMB], 0, 0, 0);
          p_share(sb, pb, ic<t>{}, ic<2 * NMB>{});
        } else {
          constexpr int t = j - 2 * NKS - 2 * NMB;
          o[t % NMB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j], pb[t / NMB], o[t % NMB], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // One tile of the step as the same fenced slot sequence (S, then P, then
    // P V): in MODE 2 a single-tile wave shares its SIMD with a PAIR wave, and
    // the fences keep its registers within the row-split step's budget.
    auto single_tile = [&](int off) {
      if constexpr (MODE == 3) {   // (MODE 3: the single-tile waves are the 16-row block's)
        narrow_scores(off, std::true_type{});
        narrow_accumulate(off, std::true_type{});
        return;
      }
      constexpr int kSlots = NKS + 2 * NMB;
      constexpr int kAhead = SDV_RS_AHEAD;
      auto operand = [&](auto jc) -> bf16x8 {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < NKS) return *(const bf16x8*)(smem + off + koff[j]);
        else return vt_operand<VKM, RG::kRowB>(lds_smem, off + ((j - NKS) / NMB) * HD * 32 + voffs[(j - NKS) % NMB]);
      };
      f32x16 sv = mneg;
      bf16x8 pv2[2];
      bf16x8 f[kSlots];
      static_for<0, kAhead>([&](auto jc) { f[decltype(jc)::value] = operand(jc); });
      static_for<0, kSlots>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j + kAhead < kSlots) f[j + kAhead] = operand(ic<j + kAhead>{});
        if constexpr (j < NKS) {
          sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j], qf[j], sv, 0, 0, 0);
          if constexpr (j == NKS - 1) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int e = 0; e < 8; ++e) pv2[ks][e] = (__bf16)fast_exp2(sv[ks * 8 + e] * p.scale_log2);
            const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pv2[ks][2 * q], pv2[ks][2 * q + 1]}, one2, l_run,
                                                        false);
            asm volatile("" ::"v"(l_run));
          }
        } else {
          constexpr int t = j - NKS;
          o[t % NMB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j], pv2[t / NMB], o[t % NMB], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto row_sum = [&]() {
      if (MODE == 3 && narrow) return row_sum4(l_run);
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
      return __uint_as_float(a[0]) + __uint_as_float(a[1]);
    };
    auto rescale = [&]() {
      if (mt > m_run + kLazy) {
        const float alpha = fast_exp2(m_run - mt);
        m_run = mt;
        m_off = -mt;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) o[mb] *= alpha;
      }
    };

    // Step k: tiles 2k and 2k+1 (PAIR waves: both; the others: tile 2k + par).
    // Wait for both, barrier, refill the stages of tiles 2k-2 and 2k-1 with
    // tiles 2k+S-2 and 2k+S-1.
    auto advance = [&](int k, int st0) {
      wait_tiles<LPW>(max(0, min(S - 4, ntiles - 2 - 2 * k)));
      if (ragged_tail && (ntiles - 1) / 2 == k) zero_tail(ntiles - 1);
      block_sync();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int tt = 2 * k + S - 2 + q;
        if (tt < ntiles) issue(tile_pages(tt), (st0 + q) % S);
      }
    };
    // Generic step (first, masked, last, and every step of the safe pass):
    // run-time stages; SAFE raises the running max lazily.
    auto tile_generic = [&](int k, int tt, int off, auto safec) {
      constexpr bool SAFE = decltype(safec)::value;
      if (wave_active && tt < ntiles) {
        scores(off, std::false_type{});
        if (k_begin + (tt + 1) * RG::kTile > N - D) mask_scores(tt);
        if constexpr (SAFE) {
          if (__any(row_max(kLazy))) rescale();
        } else if (k == 0 && (!pair || tt == 0)) {
          row_max(0.f);
          m_run = mt;
          m_off = mt == -INFINITY ? 0.f : -mt;
        }
        accumulate(off, std::false_type{});
      }
    };
    auto step_generic = [&](int k, auto safec) {
      advance(k, (2 * k + S - 2) % S);
      if constexpr (MODE == 1) {
        tile_generic(k, 2 * k, (2 * k % S) * RG::kHalf, safec);
        tile_generic(k, 2 * k + 1, ((2 * k + 1) % S) * RG::kHalf, safec);
      } else if constexpr (MODE == 0) {
        tile_generic(k, 2 * k + par, (2 * k % S) * RG::kHalf, safec);   // the parity is in koff / voffs
      } else {
        // one copy of the tile code for both roles (two inlined paths cost registers);
        // a single-tile wave's parity offset is already in koff / voffs
#pragma unroll 1
        for (int q = 0; q < 2; ++q)
          if (pair || q == par) tile_generic(k, 2 * k + q, (((2 * k + q) % S) - par) * RG::kHalf, safec);
      }
    };

    // ---- Fast pass: step 0 (reference maxima), unrolled plain steps, then the rest.
#pragma unroll
    for (int t = 0; t < S - 2; ++t)
      if (t < ntiles) issue(tile_pages(t), t);
    // plain steps: both tiles exist and need no causal mask
    const int plain = max(1, min(ntiles / 2, (N - D - k_begin) / (2 * RG::kTile)));
    const int ngroups = (plain - 1) / (S / 2);
    if (nsteps > 0) step_generic(0, std::false_type{});
#pragma unroll
    for (int e = 0; e < 16; ++e) mneg[e] = m_off / p.scale_log2;
    // (ROLE: 0 idle, 1 one tile per step, 2 both tiles)
    auto fast_steady = [&](auto rolec) {
      constexpr int ROLE = decltype(rolec)::value;
      for (int g = 0; g < ngroups; ++g) {
        const int kb = 1 + g * (S / 2);
        auto step = [&](auto uc) {
          constexpr int u = decltype(uc)::value;
          constexpr int st = (2 * (1 + u)) % S;         // stage of tile 2k (k = kb + u; kb - 1 is a multiple of S/2)
          advance(kb + u, (st + S - 2) % S);
          if constexpr (ROLE == 2) {
            if constexpr (MODE >= 2) {   // (one loop for both roles of MODES 2 and 3: the wave's role is uniform)
              if (pair) rs_pair(st * RG::kHalf, (st + 1) * RG::kHalf);
              else single_tile(st * RG::kHalf);
            } else {
              rs_pair(st * RG::kHalf, (st + 1) * RG::kHalf);
            }
          } else if constexpr (ROLE == 1) {
            scores(st * RG::kHalf, std::true_type{});
            accumulate(st * RG::kHalf, std::true_type{});
          }
        };
        step(ic<0>{});
        step(ic<1>{});
        step(ic<2>{});
        if constexpr (S > 6) step(ic<3>{});
      }
    };
    if (!wave_active) {
      fast_steady(ic<0>{});
    } else if constexpr (MODE == 0) {
      fast_steady(ic<1>{});
    } else if constexpr (MODE == 1) {
      fast_steady(ic<2>{});
    } else {
      fast_steady(ic<2>{});
    }
    for (int k = 1 + ngroups * (S / 2); k < nsteps; ++k) step_generic(k, std::false_type{});
    const bool over = wave_active && !(row_sum() <= kOverflow);

    // ---- Safe pass (only if some row's max outgrew its reference): the same
    // steps again with a running max.
    // (MODE 3: a vote per wave in LDS, the workgroup OR without a flat thread
    // index, which would otherwise be held across the item loop; a slot is
    // rewritten only in the next item, after the item's last barrier)
    int any_over = 0;
    if constexpr (MODE == 3) {
      const bool over_w = __any(over);
      if (lane == 0) s_votes[wave] = over_w ? 1 : 0;
      block_sync_lds();
#pragma unroll
      for (int w = 0; w < NW; ++w) any_over |= s_votes[w];
    } else {
      any_over = __syncthreads_or(over ? 1 : 0);
    }
    if (any_over) {
      clear();
#pragma unroll
      for (int t = 0; t < S - 2; ++t)
        if (t < ntiles) issue(tile_pages(t), t);
      for (int k = 0; k < nsteps; ++k) step_generic(k, std::true_type{});
    }
    block_sync();   // every wave is done with the ring (all loads landed: the last step waited for vmcnt 0)

    // ---- Merge the partials of the two waves of a split block: the parity-1
    // wave hands (O, l, m) to the parity-0 wave through LDS (MODE 1: every
    // wave owns its rows).
    float lt = row_sum();
    float M = partial_max(m_run, lt);
    if constexpr (MODE != 1) {
      float* xch = (float*)smem + (size_t)xslot * kMergeF * 64 + lane;
      if (giver && wave_active) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) xch[(mb * 16 + e) * 64] = o[mb][e];
        xch[(16 * NMB) * 64] = lt;
        xch[(16 * NMB + 1) * 64] = M;
      }
      block_sync_lds();
      if (!pair && !giver && wave_active && valid) {
        const float lb = xch[(16 * NMB) * 64];
        const float mb_ = xch[(16 * NMB + 1) * 64];
        const float ma = M;
        M = fmaxf(ma, mb_);
        const float wa = M == -INFINITY ? 0.f : fast_exp2(ma - M);
        const float wb = M == -INFINITY ? 0.f : fast_exp2(mb_ - M);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[mb][e] = o[mb][e] * wa + xch[(mb * 16 + e) * 64] * wb;
        lt = lt * wa + lb * wb;
      }
    }
    if (MODE == 3 && narrow && !giver && wave_active && valid) {
      // the 16-row block: lane holds query row 128 + l16 and dims 16db + 4g4 + 0..3
      const int g4 = lane_i >> 4;
      if (nsplit == 1) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const size_t obase = ((size_t)(t0 + qi) * Hq + (size_t)h * p.G + qg) * HD + g4 * 4;
#pragma unroll
        for (int db = 0; db < NDB16; ++db) {
          const int q = db % 4;
          const f32x4 v = f32x4{o[db / 4][4 * q], o[db / 4][4 * q + 1], o[db / 4][4 * q + 2], o[db / 4][4 * q + 3]} * inv;
          if (OUT_F32) {
            *(f32x4*)((float*)p.out + obase + 16 * db) = v;
          } else {
            const bf16x4 t = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            *(u32x2*)((uint16_t*)p.out + obase + 16 * db) = __builtin_bit_cast(u32x2, t);
          }
        }
      } else {
        float* slab = p.part_o + ((size_t)pslot * p.rpad + row) * HD + g4 * 4;
#pragma unroll
        for (int db = 0; db < NDB16; ++db) {
          const int q = db % 4;
          *(f32x4*)(slab + 16 * db) = f32x4{o[db / 4][4 * q], o[db / 4][4 * q + 1], o[db / 4][4 * q + 2], o[db / 4][4 * q + 3]};
        }
        if (g4 == 0) {
          float* ml = p.part_ml + ((size_t)pslot * p.rpad + row) * 2;
          ml[0] = M;
          ml[1] = lt;
        }
      }
    } else if (!giver && wave_active && valid) {
      // O^T accumulator: lane holds query row r32 and dims mb*32 + q*8 + 4hh + 0..3 in entries 4q..4q+3.
      if (nsplit == 1) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const size_t obase = ((size_t)(t0 + qi) * Hq + (size_t)h * p.G + qg) * HD + (lane_i >> 5) * 4;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = f32x4{o[mb][4 * q], o[mb][4 * q + 1], o[mb][4 * q + 2], o[mb][4 * q + 3]} * inv;
            const int dd = mb * 32 + q * 8;
            if (OUT_F32) {
              *(f32x4*)((float*)p.out + obase + dd) = v;
            } else {
              const bf16x4 t = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
              *(u32x2*)((uint16_t*)p.out + obase + dd) = __builtin_bit_cast(u32x2, t);
            }
          }
      } else {
        float* slab = p.part_o + ((size_t)pslot * p.rpad + row) * HD + (lane_i >> 5) * 4;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(f32x4*)(slab + mb * 32 + q * 8) = f32x4{o[mb][4 * q], o[mb][4 * q + 1], o[mb][4 * q + 2], o[mb][4 * q + 3]};
        if (hh == 0) {
          float* ml = p.part_ml + ((size_t)pslot * p.rpad + row) * 2;
          ml[0] = M;
          ml[1] = lt;
        }
      }
    }
    block_sync();   // the merge buffer is part of the ring
  }
}

// ---------------------------------------------------------------------------
// Merge the split-KV partials of one (sequence, KV head), 8 rows at a time:
// 32 threads per row, each thread one 4-wide slice of d.
template <int HD, int OUT_F32>
__device__ __forceinline__ void combine_rows(const AttnParams& p, int b, int h, int rblk) {
  constexpr int kRowsPerBlock = 256 / 32;
  const int chunk = p.plan[0];
  if (b < 0 || b >= p.B || chunk < 64) return;
  const int N = seq_keys(p, b);
  const int nsplit = max(1, (N + chunk - 1) / chunk);
  if (nsplit == 1) return;
  const int D = seq_drafts(p, b);
  const int R = p.G * (1 + D);
  const int row = rblk * kRowsPerBlock + (threadIdx.x >> 5);
  const int t0 = p.q_start[b];
  // (whole 32-lane groups leave together: the shuffles below stay within one group)
  if (row >= R || t0 < 0 || t0 + row / p.G >= p.total_q) return;
  const int sub = threadIdx.x & 31;
  const int item0 = p.plan[kPlanHeader + b] + h * nsplit;
  if (item0 + nsplit > p.item_cap) return;

  float M = -INFINITY;
  for (int s = sub; s < nsplit; s += 32) M = fmaxf(M, p.part_ml[((size_t)(item0 + s) * p.rpad + row) * 2]);
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 32));

  const int i = row / p.G;
  const int g = row - i * p.G;
  const size_t obase = ((size_t)(t0 + i) * p.Hkv * p.G + (size_t)h * p.G + g) * HD;
  for (int d4 = sub; d4 < HD / 4; d4 += 32) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != -INFINITY) {
      // (unrolled so that the loads of several splits are in flight together)
#pragma unroll 8
      for (int s = 0; s < nsplit; ++s) {
        const size_t slot = (size_t)(item0 + s) * p.rpad + row;
        const float ms = p.part_ml[slot * 2];
        const float w = fast_exp2(ms - M);
        L += w * p.part_ml[slot * 2 + 1];
        acc += w * *(const f32x4*)(p.part_o + slot * HD + d4 * 4);
      }
    }
    const f32x4 v = acc * (L > 0.f ? 1.f / L : 0.f);
    if (OUT_F32) {
      *(f32x4*)((float*)p.out + obase + d4 * 4) = v;
    } else {
      const bf16x4 t = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      *(u32x2*)((uint16_t*)p.out + obase + d4 * 4) = __builtin_bit_cast(u32x2, t);
    }
  }
}

// A workgroup per (sequence, KV head, block of 8 rows); unsplit sequences leave at once.
template <int HD, int OUT_F32>
__global__ __launch_bounds__(256) void verify_attn_combine(AttnParams p) {
  const int row_blocks = p.rpad / 8;
  const int unit = blockIdx.x / row_blocks;
  const int rblk = blockIdx.x - unit * row_blocks;
  const int b = unit / p.Hkv;
  combine_rows<HD, OUT_F32>(p, b, unit - b * p.Hkv, rblk);
}

// Large batches: a bounded grid walks only the sequences the plan listed as
// split (the others were written by the main kernels).
template <int HD, int OUT_F32>
__global__ __launch_bounds__(256) void verify_attn_combine_list(AttnParams p) {
  const int row_blocks = p.rpad / 8;
  const int per_seq = p.Hkv * row_blocks;
  const int* split_list = p.plan + kPlanHeader + 2 * p.B + 1;
  const int total = min(max(p.plan[3], 0), p.B) * per_seq;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int si = w / per_seq;
    const int unit = w - si * per_seq;
    const int h = unit / row_blocks;
    combine_rows<HD, OUT_F32>(p, split_list[si], h, unit - h * row_blocks);
  }
}

// ---------------------------------------------------------------------------
// Host side: variant choice, workspace layout, launches.
struct AttnLayout {
  size_t plan_off, items_off, ml_off, o_off, mask_off, total;
  int rpad, item_cap, variant;
  // variant 0: verify_attn_main, 4 waves x 16 rows (64 rows), two workgroups per CU;
  // variant 1: verify_attn_wide, 8 waves, up to 128 rows (the sets split the tiles);
  // variant 2: verify_attn_wide, 8 waves, up to 256 rows (the sets split the rows);
  // variant 3: verify_attn_wide, 8 waves, 145..192 rows (blocks 4-5 split by tile parity);
  // variant 4: verify_attn_wide, 8 waves, 129..144 rows (a 16-row block split by tile parity);
  // one workgroup per CU for variants 1 to 4
};

static int attn_variant(int rmax) {
  return rmax <= 64 ? 0 : rmax <= 128 ? 1 : rmax <= 144 ? 4 : rmax <= 192 ? 3 : 2;
}

// Resident workgroups of the persistent grid per CU.
static int attn_slots(int cus, int variant) { return cus * (variant == 0 ? 2 : 1); }

// The item cap (and so the workspace size) depends on the CU count; it is
// computed for the largest CU count of a gfx950 part so that the size query
// needs no device.
constexpr int kMaxCus = 256;
constexpr int kCombineGrid = 32 * kMaxCus;   // combine workgroups: 8 rows of one (sequence, KV head) each

// The chunk the plan is given: the caller's, or for caches no longer than the
// smallest automatic chunk that chunk itself (the plan would choose it after a
// search, and no sequence is split).
static int plan_chunk(int kv_chunk, int max_pages) {
  return kv_chunk == 0 && (long long)max_pages * kPage <= kMinChunk ? kMinChunk : kv_chunk;
}

static AttnLayout attn_layout(int B, int Hkv, int G, int HD, int max_pages, int max_draft, int kv_chunk) {
  kv_chunk = plan_chunk(kv_chunk, max_pages);
  AttnLayout L;
  const int rmax = G * (1 + max_draft);
  L.variant = attn_variant(rmax);
  L.rpad = (rmax + 15) / 16 * 16;
  const long long max_keys = (long long)max_pages * kPage;
  const long long units = (long long)B * Hkv;
  const long long slots = attn_slots(kMaxCus, L.variant);   // items the plan aims for
  long long cap;
  if (kv_chunk > 0) {
    cap = units * ((max_keys + kv_chunk - 1) / kv_chunk);
  } else {
    // the plan takes a chunk whose items fit this cap: up to kItemsPerSlot per
    // slot, and always kMaxChunk
    const long long at_max = units * ((max_keys + kMaxChunk - 1) / kMaxChunk);
    const long long at_min = units * ((max_keys + kMinChunk - 1) / kMinChunk);
    cap = std::min(at_min, std::max(slots * kItemsPerSlot, at_max));
  }
  if (cap < 1) cap = 1;
  L.item_cap = (int)cap;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.plan_off = take((size_t)(kPlanHeader + 4 * B + 1) * 4);
  L.items_off = take((size_t)cap * sizeof(ItemDesc));
  L.ml_off = take((size_t)cap * L.rpad * 2 * 4);
  L.o_off = take((size_t)cap * L.rpad * HD * 4);
  L.mask_off = take((size_t)B * (1 + max_draft) * 8);   // draft-tree masks (tree calls only)
  L.total = off;
  return L;
}

}  // namespace sdv

using namespace sdv;

size_t sdv_attn_workspace_bytes(int B, int Hkv, int G, int head_dim, int max_pages, int max_draft,
                                int kv_chunk) {
  return attn_layout(B, Hkv, G, head_dim, max_pages, max_draft, kv_chunk).total;
}

// The draft-tree mask is a template parameter, so that causal calls run code
// with no trace of it.
template <int HD, int OUTF, bool TREE, bool VKM>
static void launch_variant(int variant, const AttnParams& p, int grid, hipStream_t st) {
  if (variant == 0) verify_attn_main<HD, 1, 4, 2, OUTF, TREE, VKM><<<grid, 256, 0, st>>>(p);
  else if (variant == 1) verify_attn_wide<HD, OUTF, 0, TREE, VKM><<<grid, 512, 0, st>>>(p);
  else if (variant == 3) verify_attn_wide<HD, OUTF, 2, TREE, VKM><<<grid, 512, 0, st>>>(p);
  else if (variant == 4) verify_attn_wide<HD, OUTF, 3, TREE, VKM><<<grid, 512, 0, st>>>(p);
  else verify_attn_wide<HD, OUTF, 1, TREE, VKM><<<grid, 512, 0, st>>>(p);
}

template <int HD, int OUTF>
static void launch_main(int variant, const AttnParams& p, int grid, hipStream_t st, bool vkm) {
  if (p.tmask) {
    if (vkm) launch_variant<HD, OUTF, true, true>(variant, p, grid, st);
    else launch_variant<HD, OUTF, true, false>(variant, p, grid, st);
  } else {
    if (vkm) launch_variant<HD, OUTF, false, true>(variant, p, grid, st);
    else launch_variant<HD, OUTF, false, false>(variant, p, grid, st);
  }
}

hipError_t sdv_attn_launch(const SdAttnLaunch& a) {
  int dev = 0, cus = kMaxCus;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  cus = std::max(1, std::min(cus, kMaxCus));
  const AttnLayout L = attn_layout(a.B, a.Hkv, a.G, a.head_dim, a.max_pages, a.max_draft, a.kv_chunk);
  const int wgs = attn_slots(cus, L.variant);
  const int slots = std::max(1, wgs);   // items the plan aims for
  const int grid = (int)std::min<long long>(wgs, (long long)L.item_cap);
  unsigned char* ws = (unsigned char*)a.workspace;
  AttnParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k_cache;
  p.v = (const uint16_t*)a.v_cache;
  p.block_table = a.block_table;
  p.kv_len = a.kv_len;
  p.q_start = a.q_start;
  p.out = a.out;
  p.plan = (int*)(ws + L.plan_off);
  p.items = (ItemDesc*)(ws + L.items_off);
  p.part_ml = (float*)(ws + L.ml_off);
  p.part_o = (float*)(ws + L.o_off);
  p.B = a.B;
  p.Hkv = a.Hkv;
  p.G = a.G;
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.max_draft = a.max_draft;
  p.rpad = L.rpad;
  p.total_q = a.total_q;
  p.item_cap = L.item_cap;
  const float scale = a.softmax_scale > 0.f ? a.softmax_scale : 1.f / sqrtf((float)a.head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;

  p.tmask = nullptr;
  if (a.parents) {
    unsigned long long* masks = (unsigned long long*)(ws + L.mask_off);
    verify_tree_masks<<<(a.B + kMaskSeqsPerBlock - 1) / kMaskSeqsPerBlock, 64 * kMaskSeqsPerBlock, 0, a.stream>>>(
        p, a.parents, masks);
    p.tmask = masks;
  }
  const long long cunits = (long long)a.B * a.Hkv * (L.rpad / 8);   // combine workgroups, one per 8 rows of a head
  p.fixed_chunk = plan_chunk(a.kv_chunk, a.max_pages);
  // no sequence is longer than a fixed chunk: nothing is split, and the combine launch is left out
  const bool no_split = p.fixed_chunk > 0 && (long long)a.max_pages * kPage <= p.fixed_chunk;
  p.slots = slots;
  p.ovh_keys = kItemOverheadBytes / (4 * a.head_dim);
  p.list_splits = cunits > kCombineGrid;
  p.fused = a.B <= kFusedSeqs;   // small batches: the main kernels make the plan themselves
  if (!p.fused) {
    verify_attn_plan<<<1, kPlanThreads, 0, a.stream>>>(p, a.kv_chunk, slots, kItemOverheadBytes / (4 * a.head_dim),
                                                       p.list_splits);
    if ((long long)a.B * a.Hkv > kPlanWrites)
      verify_attn_items<<<(int)(((long long)a.B * a.Hkv + 255) / 256), 256, 0, a.stream>>>(p, p.list_splits);
  }
  if (a.head_dim == 128) {
    if (a.out_f32) launch_main<128, 1>(L.variant, p, grid, a.stream, a.v_key_major);
    else launch_main<128, 0>(L.variant, p, grid, a.stream, a.v_key_major);
  } else {
    if (a.out_f32) launch_main<64, 1>(L.variant, p, grid, a.stream, a.v_key_major);
    else launch_main<64, 0>(L.variant, p, grid, a.stream, a.v_key_major);
  }
  // one workgroup per (sequence, KV head, 8 rows), or for large batches a
  // bounded grid over the split sequences only (their number is known on the device)
  if (no_split) return hipGetLastError();
  if (cunits <= kCombineGrid) {
    const int cgrid = (int)cunits;
    if (a.head_dim == 128) {
      if (a.out_f32) verify_attn_combine<128, 1><<<cgrid, 256, 0, a.stream>>>(p);
      else verify_attn_combine<128, 0><<<cgrid, 256, 0, a.stream>>>(p);
    } else {
      if (a.out_f32) verify_attn_combine<64, 1><<<cgrid, 256, 0, a.stream>>>(p);
      else verify_attn_combine<64, 0><<<cgrid, 256, 0, a.stream>>>(p);
    }
  } else {
    if (a.head_dim == 128) {
      if (a.out_f32) verify_attn_combine_list<128, 1><<<kCombineGrid, 256, 0, a.stream>>>(p);
      else verify_attn_combine_list<128, 0><<<kCombineGrid, 256, 0, a.stream>>>(p);
    } else {
      if (a.out_f32) verify_attn_combine_list<64, 1><<<kCombineGrid, 256, 0, a.stream>>>(p);
      else verify_attn_combine_list<64, 0><<<kCombineGrid, 256, 0, a.stream>>>(p);
    }
  }
  return hipGetLastError();
}
