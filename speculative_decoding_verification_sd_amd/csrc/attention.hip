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
// plan kernel picks the smallest chunk (a multiple of 64 keys) whose item
// count fits the resident workgroups of the grid, so that every item runs
// concurrently, and writes one descriptor per item.  A persistent grid walks
// the items.
//
// Per item, a workgroup of NW waves runs over 32-key tiles (two 16-key pages):
//   * K and V tiles travel global -> LDS with global_load_lds_dwordx4 (no
//     registers) into a ring of kStages tiles, paced by explicit vmcnt waits
//     and a bare s_barrier, so kStages-1 tiles are in flight per workgroup.
//     LDS rows are XOR-swizzled in 16-byte chunks against bank conflicts.
//   * Each wave owns NRB blocks of 16 query rows.  S^T = K * Q^T is computed
//     with v_mfma_f32_16x16x32_bf16 (Q stays in registers), so each lane holds
//     one query row: the online softmax reduces across four lanes with
//     v_permlane32_swap / v_permlane16_swap, and the running max is raised
//     lazily (only when it grows by more than 2^8), which leaves the output
//     rescale out of almost every tile.
//   * P (bf16) is taken straight from the S^T accumulators as the B operand
//     of O^T = V^T * P^T; V is read transposed with ds_read_b64_tr_b16 in the
//     same key order.
// Items that cover a whole sequence write the output; otherwise the
// unnormalised partial (O, m, l) goes to the workspace and a combine kernel
// merges the splits with their log-sum-exp weights.

#include <math.h>

#include <algorithm>

#include "common.h"

namespace sdv {

constexpr int kPage = 16;
constexpr int kMinChunk = 256;
constexpr int kMaxChunk = 16384;         // keys per work item; bounds the per-item page list in LDS
constexpr int kPlanThreads = 256;
constexpr int kPlanHeader = 4;

// Ring depth (tiles resident in LDS per workgroup).  Build-time tunables: the
// 4-wave variants run two workgroups per CU, the 8-wave one a single one.
#ifndef SDV_RING_STAGES
#define SDV_RING_STAGES 3
#endif
#ifndef SDV_RING_STAGES_WIDE
#define SDV_RING_STAGES_WIDE 6
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
  int* plan;        // [4 + B + 1]: chunk, total items, -, -, item_start[0..B]
  ItemDesc* items;  // [item_cap]
  int B, Hkv, G, max_pages, num_pages, max_draft, rpad, total_q, item_cap;
  float scale_log2;
};

__device__ __forceinline__ int seq_keys(const AttnParams& p, int b) {
  return min(max(p.kv_len[b], 0), p.max_pages * kPage);
}

__device__ __forceinline__ int seq_drafts(const AttnParams& p, int b) {
  return min(max(p.q_start[b + 1] - p.q_start[b] - 1, 0), p.max_draft);
}

// ---------------------------------------------------------------------------
// Plan (one workgroup).  Chunk: `fixed_chunk` if non-zero, else the smallest
// multiple of 64 in [kMinChunk, kMaxChunk] whose item count
// Hkv * sum_b max(1, ceil(N_b / chunk)) fits `slots` (thread t evaluates
// chunk kMinChunk + 64 t).  Then the exclusive prefix of items per sequence
// and one descriptor per item.
__global__ __launch_bounds__(kPlanThreads) void verify_attn_plan(AttnParams p, int fixed_chunk, int slots) {
  __shared__ int s_keys[kPlanThreads];
  __shared__ int scan[kPlanThreads];
  __shared__ int s_best;
  const int tid = threadIdx.x;
  const int max_keys = p.max_pages * kPage;
  const int cap_chunk = max(kMinChunk, min(kMaxChunk, (max_keys + 63) / 64 * 64));
  const int my_chunk = min(kMinChunk + 64 * tid, cap_chunk);
  long long my_items = 0;
  for (int base = 0; base < p.B; base += kPlanThreads) {
    __syncthreads();
    s_keys[tid] = base + tid < p.B ? seq_keys(p, base + tid) : 0;
    __syncthreads();
    const int n = min(kPlanThreads, p.B - base);
    for (int j = 0; j < n; ++j) my_items += max(1, (s_keys[j] + my_chunk - 1) / my_chunk);
  }
  if (tid == 0) s_best = cap_chunk;
  __syncthreads();
  if (my_items * p.Hkv <= slots) atomicMin(&s_best, my_chunk);
  __syncthreads();
  const int chunk = fixed_chunk > 0 ? fixed_chunk : s_best;

  int carry = 0;
  for (int base = 0; base < p.B; base += kPlanThreads) {
    const int b = base + tid;
    int v = 0, N = 0, ns = 1;
    if (b < p.B) {
      N = seq_keys(p, b);
      ns = max(1, (N + chunk - 1) / chunk);
      v = ns * p.Hkv;
    }
    scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int first = carry + scan[tid] - v;
    if (b < p.B) {
      p.plan[kPlanHeader + b] = first;
      const int t0 = p.q_start[b];
      const int D = seq_drafts(p, b);
      for (int h = 0; h < p.Hkv; ++h)
        for (int s = 0; s < ns; ++s) {
          const int it = first + h * ns + s;
          if (it < p.item_cap) {
            ItemDesc d;
            d.b = b;
            d.h = h;
            d.k_begin = s * chunk;
            d.k_end = min(N, (s + 1) * chunk);
            d.t0 = t0;
            d.D = D;
            d.N = N;
            d.nsplit = ns;
            p.items[it] = d;
          }
        }
    }
    carry += scan[kPlanThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    p.plan[0] = chunk;
    p.plan[1] = carry;
    p.plan[kPlanHeader + p.B] = carry;
  }
}

// ---------------------------------------------------------------------------
// Wait until at most N vector-memory operations of this wave are in flight
// (LDS-DMA loads count like any other vector load).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt immediate: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// XOR swizzle of the 16-byte chunk index inside a K or V row of the LDS tile,
// as a function of the key's position mod 16, for 64 banks of 4 bytes: the
// 16 lanes of a ds_read_b128 (K operand, sixteen keys at one logical chunk)
// and the 32 lanes of a ds_read_b64_tr_b16 (eight keys, two adjacent chunks)
// each touch every bank at most once.
template <int HD>
__device__ __forceinline__ int chunk_swz(int k) {
  if constexpr (HD == 128) return ((k & 7) << 1) | ((k >> 3) & 1);
  else return (((k >> 1) & 3) << 1) | ((k >> 3) & 1);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// One 16-byte-per-lane global->LDS DMA (global_load_lds_dwordx4, scalar-base
// form): lane i reads base + voff_i and its 16 bytes land at LDS byte address
// lds_addr + 16*i; base and lds_addr are wave-uniform (lds_addr goes to M0).
// Issued as inline asm so that the compiler's waitcount logic does not pace
// every later LDS read on these loads (it cannot tell ring stages apart and
// would wait for all of them); the ring waits for them explicitly with
// s_waitcnt vmcnt before its barrier.  M0 is written only here in this
// kernel, which a build test checks on the generated ISA.
__device__ __forceinline__ void dma16(const unsigned char* base, unsigned voff, unsigned lds_addr) {
  // readfirstlane returns int: go through unsigned so the low word is zero-extended
  const uint64_t b = (uint64_t)base;
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sb)
               : "memory", "m0");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

template <int HD, int NW>
struct Ring {
  static constexpr int kTile = 32;                        // keys per tile (two pages)
  static constexpr int kRowB = HD * 2;                    // bytes per key row
  static constexpr int kCpr = kRowB / 16;                 // 16-byte chunks per row
  static constexpr int kHalf = kTile * kRowB;             // K (or V) bytes per tile
  static constexpr int kStageB = 2 * kHalf;
  static constexpr int kStages = NW >= 8 ? SDV_RING_STAGES_WIDE : SDV_RING_STAGES;
  static constexpr int kLoadsKV = 2 * kHalf / 1024;       // 1 KB DMA instructions per tile (K and V)
  static constexpr int kLPW = kLoadsKV / NW;              // ... per wave
  static constexpr int kKeysPerLoad = 1024 / kRowB;       // key rows one instruction fills
  static_assert(kStages >= 2 && kStages <= 8, "ring depth");
  static_assert(kLoadsKV % NW == 0 && kLPW >= 1, "DMA instructions divide evenly over the waves");
};

// ---------------------------------------------------------------------------
template <int HD, int NRB, int NW, int OUT_F32>
__global__ __launch_bounds__(64 * NW, (NW >= 8 ? 1 : 2)) void verify_attn_main(AttnParams p) {
  using RG = Ring<HD, NW>;
  constexpr int NKC = HD / 32;   // MFMA k-steps over d for S
  constexpr int NDB = HD / 16;   // 16-wide d blocks of O
  constexpr int LPW = RG::kLPW;
  constexpr int kPageB = kPage * HD * 2;   // bytes of one (page, head) block
  constexpr float kLazy = 8.f;             // raise the running max only when it grows by more than 2^8
  constexpr int kPageSlots = kMaxChunk / kPage + 2;
  // one LDS object: the K/V ring followed by the page ids of the current item
  __shared__ __attribute__((aligned(1024))) unsigned char smem[RG::kStages * RG::kStageB + kPageSlots * 4];
  int* s_pages = (int*)(smem + RG::kStages * RG::kStageB);
  lds_u8* lds_smem = (lds_u8*)smem;
  const unsigned lds_base = (unsigned)(size_t)lds_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int total = min(p.plan[1], p.item_cap);
  const int Hq = p.Hkv * p.G;

  // lane-constant offsets
  const int kswz = chunk_swz<HD>(l16) & (RG::kCpr - 1);                   // K operand: key = kb*16 + l16
  const int vkey = g4 * 4 + (l16 >> 2);                               // transposed V read: key row
  const int vswz = chunk_swz<HD>(vkey) & (RG::kCpr - 1);
  const int vsub = (l16 & 3) >> 1;                                    // chunk within the 16-wide d block
  const int vbyte = (l16 & 1) * 8;
  // DMA instruction j = wave + NW*i of a tile: K rows for j < kLoadsKV/2, V rows after
  unsigned dma_off[LPW];         // byte offset of this lane's 16 bytes inside the (page, head) block
  int dma_row[LPW];              // first key row (tile-relative) the instruction fills
  int dma_kv[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave + NW * i;
    dma_kv[i] = j >= RG::kLoadsKV / 2;
    dma_row[i] = (j % (RG::kLoadsKV / 2)) * RG::kKeysPerLoad;
    const int key = dma_row[i] + lane / RG::kCpr;
    const int lc = (lane % RG::kCpr) ^ (chunk_swz<HD>(key & 15) & (RG::kCpr - 1));
    dma_off[i] = (unsigned)(((key & 15) * HD + lc * 8) * 2);
  }

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const ItemDesc d = p.items[item];
    const int b = d.b, h = d.h, k_begin = d.k_begin, k_end = d.k_end;
    const int t0 = d.t0, D = d.D, N = d.N, nsplit = d.nsplit;
    const int R = p.G * (1 + D);
    const int* bt = p.block_table + (size_t)b * p.max_pages;
    const bool wave_active = wave * NRB * 16 < R;
    const int ntiles = k_end > k_begin ? (k_end - k_begin + RG::kTile - 1) / RG::kTile : 0;
    const unsigned char* kbase = (const unsigned char*)p.k + (size_t)h * kPageB;
    const unsigned char* vbase = (const unsigned char*)p.v + (size_t)h * kPageB;
    const size_t page_stride = (size_t)p.Hkv * kPageB;

    // Issue this wave's share of the LDS-DMA loads of tile `tile` into its ring stage.
    auto issue = [&](int tile) {
      const unsigned st = lds_base + (unsigned)((tile % RG::kStages) * RG::kStageB);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        // the rows of one instruction lie in one page
        const int pid = __builtin_amdgcn_readfirstlane(s_pages[tile * (RG::kTile / kPage) + dma_row[i] / kPage]);
        dma16((dma_kv[i] ? vbase : kbase) + (size_t)pid * page_stride, dma_off[i],
              st + (unsigned)(dma_kv[i] * RG::kHalf + dma_row[i] * RG::kRowB));
      }
    };

    // Query fragments (B operand of S^T = K Q^T): lane holds row l16, dims g4*8..+7 of each 32-wide step.
    bf16x8 qf[NRB][NKC];
    int pos[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = (wave * NRB + rb) * 16 + l16;
      const int i0 = row / p.G;
      const bool valid = row < R && t0 >= 0 && t0 + i0 < p.total_q;
      const int i = valid ? i0 : 0;
      const int g = valid ? row - i * p.G : 0;
      pos[rb] = valid ? N - 1 - D + i : -1;
      const uint16_t* qp = p.q + ((size_t)(t0 + i) * Hq + (size_t)h * p.G + g) * HD + g4 * 8;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        u32x4 raw = valid ? *(const u32x4*)(qp + c * 32) : u32x4{0, 0, 0, 0};
        qf[rb][c] = __builtin_bit_cast(bf16x8, raw);
      }
    }

    float m_run[NRB], l_run[NRB];
    f32x4 o[NRB][NDB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      m_run[rb] = -INFINITY;
      l_run[rb] = 0.f;
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
    wait_lds();
    block_sync();
#pragma unroll
    for (int t = 0; t < RG::kStages - 1; ++t)
      if (t < ntiles) issue(t);

    auto compute = [&](int tile) {
      const unsigned char* Ks = smem + (tile % RG::kStages) * RG::kStageB;
      const int ts = k_begin + tile * RG::kTile;
      const bool need_mask = ts + RG::kTile > N - D;

      f32x4 sc[2][NRB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 kf[NKC];
        const unsigned char* krow = Ks + (kb * 16 + l16) * RG::kRowB;
#pragma unroll
        for (int c = 0; c < NKC; ++c) kf[c] = *(const bf16x8*)(krow + (((c * 4 + g4) ^ kswz) * 16));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NKC; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[rb][c], acc, 0, 0, 0);
          sc[kb][rb] = acc;
        }
      }

      // online softmax, one query row per lane; lazy rescale of the running max
      float mt[NRB];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (ts + kb * 16 + g4 * 4 + e > pos[rb]) sc[kb][rb][e] = -INFINITY;
        }
        float m = fmaxf(fmaxf(sc[0][rb][0], sc[0][rb][1]), fmaxf(sc[0][rb][2], sc[0][rb][3]));
        m = fmaxf(m, fmaxf(fmaxf(sc[1][rb][0], sc[1][rb][1]), fmaxf(sc[1][rb][2], sc[1][rb][3])));
        mt[rb] = row_max4(m) * p.scale_log2;
        grow |= mt[rb] > m_run[rb] + kLazy;
      }
      if (__any(grow)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          if (mt[rb] > m_run[rb] + kLazy) {
            const float alpha = fast_exp2(m_run[rb] - mt[rb]);
            m_run[rb] = mt[rb];
            l_run[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[rb][db] *= alpha;
          }
        }
      }
      bf16x8 pf[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mc = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
        float psum = 0.f;
        bf16x8 t;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = fast_exp2(fmaf(sc[kb][rb][e], p.scale_log2, -mc));
            psum += pv;
            t[kb * 4 + e] = (__bf16)pv;
          }
        l_run[rb] += psum;
        pf[rb] = t;
      }

      // O^T += V^T P^T: V read transposed from LDS, keys in the order of the S^T accumulators
      const int vstage = (tile % RG::kStages) * RG::kStageB + RG::kHalf + vkey * RG::kRowB + vbyte;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int voff = vstage + (((db * 2 + vsub) ^ vswz) * 16);
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_smem + voff));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_smem + voff + 16 * RG::kRowB));
        const u32x2 lo = __builtin_bit_cast(u32x2, lo4);
        const u32x2 hi = __builtin_bit_cast(u32x2, hi4);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], o[rb][db], 0, 0, 0);
      }
    };

    // steady state: every iteration has kStages-2 younger tiles in flight and issues one more
    const int nsteady = ntiles - (RG::kStages - 1);
    int tile = 0;
    for (; tile < nsteady; ++tile) {
      wait_vmem<(RG::kStages - 2) * LPW>();
      block_sync();
      issue(tile + RG::kStages - 1);
      if (wave_active) compute(tile);
    }
    // drain: the last kStages-1 tiles are all in flight already
    for (; tile < ntiles; ++tile) {
      switch (ntiles - 1 - tile) {
        case 6: wait_vmem<6 * LPW>(); break;
        case 5: wait_vmem<5 * LPW>(); break;
        case 4: wait_vmem<4 * LPW>(); break;
        case 3: wait_vmem<3 * LPW>(); break;
        case 2: wait_vmem<2 * LPW>(); break;
        case 1: wait_vmem<LPW>(); break;
        default: wait_vmem<0>(); break;
      }
      if (k_begin + (tile + 1) * RG::kTile > k_end) {
        // zero the key rows at or past k_end that this wave loaded (last tile only)
        unsigned char* st = smem + (tile % RG::kStages) * RG::kStageB;
        const int ts = k_begin + tile * RG::kTile;
#pragma unroll
        for (int i = 0; i < LPW; ++i)
          if (ts + dma_row[i] + lane / RG::kCpr >= k_end)
            *(u32x4*)(st + dma_kv[i] * RG::kHalf + dma_row[i] * RG::kRowB + lane * 16) = u32x4{0, 0, 0, 0};
        wait_lds();
      }
      block_sync();
      if (wave_active) compute(tile);
    }
    // every wave is done with the ring before the next item's loads land in it
    block_sync();

    if (wave_active) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float lt = row_sum4(l_run[rb]);
        const int row = (wave * NRB + rb) * 16 + l16;
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
          float* slab = p.part_o + ((size_t)item * p.rpad + row) * HD + g4 * 4;
#pragma unroll
          for (int db = 0; db < NDB; ++db) *(f32x4*)(slab + db * 16) = o[rb][db];
          if (g4 == 0) {
            float* ml = p.part_ml + ((size_t)item * p.rpad + row) * 2;
            ml[0] = m_run[rb];
            ml[1] = lt;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge the split-KV partials of one (sequence, KV head): 8 rows per
// workgroup, 32 threads per row, each thread one 4-wide slice of d.
template <int HD, int OUT_F32>
__global__ __launch_bounds__(256) void verify_attn_combine(AttnParams p) {
  constexpr int kRowsPerBlock = 256 / 32;
  const int row_blocks = p.rpad / kRowsPerBlock;
  const int unit = blockIdx.x / row_blocks;
  const int rblk = blockIdx.x - unit * row_blocks;
  const int b = unit / p.Hkv;
  const int h = unit - b * p.Hkv;
  const int chunk = p.plan[0];
  const int N = seq_keys(p, b);
  const int nsplit = max(1, (N + chunk - 1) / chunk);
  if (nsplit == 1) return;
  const int D = seq_drafts(p, b);
  const int R = p.G * (1 + D);
  const int row = rblk * kRowsPerBlock + (threadIdx.x >> 5);
  const int t0 = p.q_start[b];
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

// ---------------------------------------------------------------------------
// Host side: variant choice, workspace layout, launches.
struct AttnLayout {
  size_t plan_off, items_off, ml_off, o_off, total;
  int rpad, item_cap, variant;   // variant 0: 1 row block x 4 waves, 1: 2 x 4, 2: 2 x 8
};

static int attn_variant(int rmax) { return rmax <= 64 ? 0 : (rmax <= 128 ? 1 : 2); }

// Resident workgroups of the persistent grid per CU (the plan targets that many items).
static int attn_slots(int cus, int variant) { return cus * (variant == 2 ? 1 : 2); }

// The item cap (and so the workspace size) depends on the CU count; it is
// computed for the largest CU count of a gfx950 part so that the size query
// needs no device.
constexpr int kMaxCus = 256;

static AttnLayout attn_layout(int B, int Hkv, int G, int HD, int max_pages, int max_draft, int kv_chunk) {
  AttnLayout L;
  const int rmax = G * (1 + max_draft);
  L.variant = attn_variant(rmax);
  L.rpad = (rmax + 15) / 16 * 16;
  const long long max_keys = (long long)max_pages * kPage;
  const long long units = (long long)B * Hkv;
  const long long slots = attn_slots(kMaxCus, L.variant);
  long long cap;
  if (kv_chunk > 0) {
    cap = units * ((max_keys + kv_chunk - 1) / kv_chunk);
  } else {
    // the plan picks the smallest chunk with at most `slots` items, else kMaxChunk
    const long long at_max = units * ((max_keys + kMaxChunk - 1) / kMaxChunk);
    const long long at_min = units * ((max_keys + kMinChunk - 1) / kMinChunk);
    cap = std::min(at_min, std::max(slots, at_max));
  }
  if (cap < 1) cap = 1;
  L.item_cap = (int)cap;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.plan_off = take((size_t)(kPlanHeader + B + 1) * 4);
  L.items_off = take((size_t)cap * sizeof(ItemDesc));
  L.ml_off = take((size_t)cap * L.rpad * 2 * 4);
  L.o_off = take((size_t)cap * L.rpad * HD * 4);
  L.total = off;
  return L;
}

}  // namespace sdv

using namespace sdv;

size_t sdv_attn_workspace_bytes(int B, int Hkv, int G, int head_dim, int max_pages, int max_draft,
                                int kv_chunk) {
  return attn_layout(B, Hkv, G, head_dim, max_pages, max_draft, kv_chunk).total;
}

template <int HD, int OUTF>
static void launch_main(int variant, const AttnParams& p, int grid, hipStream_t st) {
  if (variant == 0) verify_attn_main<HD, 1, 4, OUTF><<<grid, 256, 0, st>>>(p);
  else if (variant == 1) verify_attn_main<HD, 2, 4, OUTF><<<grid, 256, 0, st>>>(p);
  else verify_attn_main<HD, 2, 8, OUTF><<<grid, 512, 0, st>>>(p);
}

hipError_t sdv_attn_launch(const SdAttnLaunch& a) {
  int dev = 0, cus = kMaxCus;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  cus = std::max(1, std::min(cus, kMaxCus));
  const AttnLayout L = attn_layout(a.B, a.Hkv, a.G, a.head_dim, a.max_pages, a.max_draft, a.kv_chunk);
  const int slots = (int)std::min<long long>(attn_slots(cus, L.variant), L.item_cap);
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

  verify_attn_plan<<<1, kPlanThreads, 0, a.stream>>>(p, a.kv_chunk, slots);
  if (a.head_dim == 128) {
    if (a.out_f32) launch_main<128, 1>(L.variant, p, slots, a.stream);
    else launch_main<128, 0>(L.variant, p, slots, a.stream);
  } else {
    if (a.out_f32) launch_main<64, 1>(L.variant, p, slots, a.stream);
    else launch_main<64, 0>(L.variant, p, slots, a.stream);
  }
  const int cgrid = a.B * a.Hkv * (L.rpad / 8);
  if (a.head_dim == 128) {
    if (a.out_f32) verify_attn_combine<128, 1><<<cgrid, 256, 0, a.stream>>>(p);
    else verify_attn_combine<128, 0><<<cgrid, 256, 0, a.stream>>>(p);
  } else {
    if (a.out_f32) verify_attn_combine<64, 1><<<cgrid, 256, 0, a.stream>>>(p);
    else verify_attn_combine<64, 0><<<cgrid, 256, 0, a.stream>>>(p);
  }
  return hipGetLastError();
}
