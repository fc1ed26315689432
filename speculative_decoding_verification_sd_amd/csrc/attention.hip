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
// Work decomposition (split-KV): a sequence's keys are cut into chunks of
// `chunk` keys (a multiple of the 64-key tile); a work item is
// (sequence, KV head, chunk).  The chunk size is picked on the device from the
// batch's total key count so that ragged batches give evenly sized items.
// A persistent grid (a few workgroups per CU) walks the item list.
//
// Per item, a 256-thread workgroup (4 waves) runs over 64-key tiles:
//   * K and V tiles (4 pages of 16 keys) are gathered through the block table
//     with 16-byte loads, prefetched into registers one tile ahead and staged
//     in LDS (double buffer).  K is kept row-major (padded rows); V is written
//     transposed (d-major, XOR-swizzled 8-byte slots) so that PV operands are
//     8-byte LDS reads.
//   * Each wave owns NRB blocks of 16 query rows.  S^T = K * Q^T is computed
//     with v_mfma_f32_16x16x32_bf16 (Q stays in registers), so each lane ends
//     up holding one query row: the online softmax needs only two cross-lane
//     max steps per tile and the output rescale is lane-local.
//   * P (bf16) is reused straight from the S^T accumulators as the B operand
//     of O^T = V^T * P^T (key order inside each 32-key block permuted to match
//     the accumulator layout; V is read in the same order).
// Items that cover a whole sequence write the output; otherwise the
// unnormalised partial (O, m, l) goes to the workspace and a combine kernel
// merges the splits with their log-sum-exp weights.

#include <math.h>

#include "common.h"

namespace sdv {

constexpr int kPage = 16;
constexpr int kTileKeys = 64;
constexpr int kThreads = 256;
constexpr int kMinChunk = 256;
constexpr int kMaxChunk = 8192;          // keys per work item; bounds the per-item page list in LDS
constexpr int kTargetItems = 1024;
constexpr int kPlanHeader = 4;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int* block_table;
  const int* kv_len;
  const int* q_start;
  void* out;
  float* part_o;   // [item_cap, rpad, d]   unnormalised partial outputs
  float* part_ml;  // [item_cap, rpad, 2]   (running max in log2 units, sum)
  int* plan;       // [4 + B + 1]: chunk, total items, -, -, item_start[0..B]
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
// Plan: chunk size and the exclusive prefix of work items per sequence.
__global__ __launch_bounds__(kThreads) void verify_attn_plan(AttnParams p, int fixed_chunk) {
  __shared__ long long red[kThreads];
  __shared__ int scan[kThreads];
  __shared__ int s_chunk;
  const int tid = threadIdx.x;
  long long tot = 0;
  for (int b = tid; b < p.B; b += kThreads) tot += seq_keys(p, b);
  red[tid] = tot;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    int chunk = fixed_chunk;
    if (chunk <= 0) {
      long long want = (red[0] * p.Hkv + kTargetItems - 1) / kTargetItems;
      want = (want + kTileKeys - 1) / kTileKeys * kTileKeys;
      const long long cap = ((long long)p.max_pages * kPage + kTileKeys - 1) / kTileKeys * kTileKeys;
      chunk = (int)min(min(cap, (long long)kMaxChunk), max((long long)kMinChunk, want));
    }
    s_chunk = chunk;
  }
  __syncthreads();
  const int chunk = s_chunk;
  int carry = 0;
  for (int base = 0; base < p.B; base += kThreads) {
    const int b = base + tid;
    int v = 0;
    if (b < p.B) v = max(1, (seq_keys(p, b) + chunk - 1) / chunk) * p.Hkv;
    scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    if (b < p.B) p.plan[kPlanHeader + b] = carry + scan[tid] - v;
    carry += scan[kThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    p.plan[0] = chunk;
    p.plan[1] = carry;
    p.plan[kPlanHeader + p.B] = carry;
  }
}

// Wait until at most `n` vector-memory operations of this wave are in flight
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
// as a function of the key's position mod 16.  Eight consecutive keys read at
// one logical chunk (K operand) and four consecutive keys read at two adjacent
// chunks (transposed V reads) both land on distinct bank groups.
__device__ __forceinline__ int chunk_swz(int k) {
  return ((k & 3) << 1) ^ ((k >> 2) & 1) ^ (((k >> 3) & 1) << 3);
}

// One 16-byte-per-lane global->LDS DMA (global_load_lds_dwordx4): lane i's 16 bytes land
// at LDS byte address lds_addr + 16*i (lds_addr is wave-uniform, passed in M0).  Issued as
// inline asm so that the compiler does not pace LDS reads on these loads; the ring below
// waits for them explicitly with s_waitcnt vmcnt before a barrier.
__device__ __forceinline__ void dma16(const void* src, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
               : "memory", "m0");
}

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int HD, int NRB>
struct Ring {
  static constexpr int kTile = 32;                       // keys per tile (two pages)
  static constexpr int kRowB = HD * 2;                   // bytes per key row
  static constexpr int kCpr = kRowB / 16;                // 16-byte chunks per row
  static constexpr int kHalf = kTile * kRowB;            // K (or V) bytes per tile
  static constexpr int kStageB = 2 * kHalf;
  static constexpr int kStages = NRB >= 4 ? 8 : 4;       // ring depth
  static constexpr int kLoadsPerWave = kHalf / 1024 / 4; // DMA instructions per wave for K (same for V)
  static constexpr int kKeysPerLoad = 1024 / kRowB;      // key rows one wave instruction fills
};

// ---------------------------------------------------------------------------
template <int HD, int NRB, int OUT_F32>
__global__ __launch_bounds__(kThreads, (NRB >= 4 ? 1 : 2)) void verify_attn_main(AttnParams p) {
  using RG = Ring<HD, NRB>;
  constexpr int NKC = HD / 32;   // MFMA k-steps over d for S
  constexpr int NDB = HD / 16;   // 16-wide d blocks of O
  constexpr int LPW = 2 * RG::kLoadsPerWave;
  constexpr float kLazy = 8.f;   // rescale only when a row max grows by more than 2^8
  // one LDS object: the K/V ring followed by the page ids of the current item
  __shared__ __attribute__((aligned(1024))) unsigned char smem[RG::kStages * RG::kStageB +
                                                              (kMaxChunk / kPage + 2) * 4];
  int* s_pages = (int*)(smem + RG::kStages * RG::kStageB);
  __attribute__((address_space(3))) unsigned char* lds_smem = (__attribute__((address_space(3))) unsigned char*)smem;
  const unsigned lds_base = (unsigned)(size_t)lds_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int chunk = p.plan[0];
  const int total = min(p.plan[1], p.item_cap);
  const int* item_start = p.plan + kPlanHeader;
  const int Hq = p.Hkv * p.G;

  // lane-constant LDS offsets
  const int kswz = chunk_swz(l16) & (RG::kCpr - 1);                   // K operand: key = kb*16 + l16
  const int vkey = g4 * 4 + (l16 >> 2);                               // transposed V read: key row
  const int vswz = chunk_swz(vkey) & (RG::kCpr - 1);
  const int vsub = (l16 & 3) >> 1;                                    // chunk within the 16-wide d block
  const int vbyte = (l16 & 1) * 8;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (item_start[mid] <= item) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int N = seq_keys(p, b);
    const int nsplit = max(1, (N + chunk - 1) / chunk);
    const int local = item - item_start[b];
    const int h = local / nsplit;
    const int s = local - h * nsplit;
    const int t0 = p.q_start[b];
    const int D = seq_drafts(p, b);
    const int R = p.G * (1 + D);
    const int k_begin = s * chunk;
    const int k_end = min(N, k_begin + chunk);
    const int* bt = p.block_table + (size_t)b * p.max_pages;
    const bool wave_active = wave * NRB * 16 < R;
    const int ntiles = k_end > k_begin ? (k_end - k_begin + RG::kTile - 1) / RG::kTile : 0;
    static_assert(kMaxChunk % RG::kTile == 0, "tiles never straddle an item");

    // Issue this wave's share of the LDS-DMA loads of tile `tile` into its ring stage.
    auto issue = [&](int tile) {
      const int ts = k_begin + tile * RG::kTile;
      unsigned char* st = smem + (tile % RG::kStages) * RG::kStageB;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        const uint16_t* cache = kv ? p.v : p.k;
#pragma unroll
        for (int i = 0; i < RG::kLoadsPerWave; ++i) {
          // the rows one instruction fills lie in one page
          const int row0 = (wave * RG::kLoadsPerWave + i) * RG::kKeysPerLoad;
          const int pid = s_pages[tile * (RG::kTile / kPage) + row0 / kPage];
          const int key = row0 + lane / RG::kCpr;
          const int pc = lane % RG::kCpr;
          const int lc = pc ^ (chunk_swz(key & 15) & (RG::kCpr - 1));
          const int gk = ts + key;
          // keys past the end read a valid dummy chunk and are zeroed in LDS before use
          const uint16_t* src = gk < k_end
              ? cache + (((size_t)pid * p.Hkv + h) * kPage + (gk & (kPage - 1))) * HD + lc * 8
              : cache;
          dma16(src, lds_base + (unsigned)((st - smem) + kv * RG::kHalf + row0 * RG::kRowB));
        }
      }
    };
    // Zero the key rows of tile `tile` at or past k_end that this wave loaded.
    auto zero_tail = [&](int tile) {
      const int ts = k_begin + tile * RG::kTile;
      unsigned char* st = smem + (tile % RG::kStages) * RG::kStageB;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
#pragma unroll
        for (int i = 0; i < RG::kLoadsPerWave; ++i) {
          const int row0 = (wave * RG::kLoadsPerWave + i) * RG::kKeysPerLoad;
          if (ts + row0 + lane / RG::kCpr >= k_end)
            *(u32x4*)(st + kv * RG::kHalf + row0 * RG::kRowB + lane * 16) = u32x4{0, 0, 0, 0};
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

    // page ids of this item (clamped into the pool), then drain every load issued so far so
    // that the ring's vmcnt accounting below only ever sees its own LDS-DMA loads
    const int page0 = k_begin / kPage;
    const int npages = (k_end + kPage - 1) / kPage - page0;
    for (int j = tid; j < npages; j += kThreads) s_pages[j] = min(max(bt[page0 + j], 0), p.num_pages - 1);
    wait_vmem<0>();
    wait_lds();
    block_sync();
#pragma unroll
    for (int t = 0; t < RG::kStages - 1; ++t)
      if (t < ntiles) issue(t);

    for (int tile = 0; tile < ntiles; ++tile) {
      // tiles issued after this one: tile+1 .. min(ntiles-1, tile+kStages-2)
      const int after = min(RG::kStages - 2, ntiles - 1 - tile);
      if constexpr (RG::kStages == 4) {
        if (after >= 2) wait_vmem<2 * LPW>();
        else if (after == 1) wait_vmem<LPW>();
        else wait_vmem<0>();
      } else {
        switch (after) {
          case 6: wait_vmem<6 * LPW>(); break;
          case 5: wait_vmem<5 * LPW>(); break;
          case 4: wait_vmem<4 * LPW>(); break;
          case 3: wait_vmem<3 * LPW>(); break;
          case 2: wait_vmem<2 * LPW>(); break;
          case 1: wait_vmem<LPW>(); break;
          default: wait_vmem<0>(); break;
        }
      }
      const int ts = k_begin + tile * RG::kTile;
      if (ts + RG::kTile > k_end) {
        zero_tail(tile);
        wait_lds();
      }
      block_sync();
      if (tile + RG::kStages - 1 < ntiles) issue(tile + RG::kStages - 1);

      if (wave_active) {
        const unsigned char* Ks = smem + (tile % RG::kStages) * RG::kStageB;
        const unsigned char* Vs = Ks + RG::kHalf;
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
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          mt[rb] = m * p.scale_log2;
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
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int pc = (db * 2 + vsub) ^ vswz;
          const int voff = (tile % RG::kStages) * RG::kStageB + RG::kHalf + vkey * RG::kRowB + pc * 16 + vbyte;
          const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_smem + voff));
          const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_smem + voff + 16 * RG::kRowB));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, u32x4{__builtin_bit_cast(u32x2, lo4)[0], __builtin_bit_cast(u32x2, lo4)[1],
                            __builtin_bit_cast(u32x2, hi4)[0], __builtin_bit_cast(u32x2, hi4)[1]});
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], o[rb][db], 0, 0, 0);
        }
      }
    }
    // every wave is done with the ring before the next item's loads land in it
    block_sync();

    if (wave_active) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float lt = l_run[rb] + __shfl_xor(l_run[rb], 16);
        lt += __shfl_xor(lt, 32);
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
__global__ __launch_bounds__(kThreads) void verify_attn_combine(AttnParams p) {
  constexpr int kRowsPerBlock = kThreads / 32;
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
struct AttnLayout {
  size_t plan_off, ml_off, o_off, total;
  int rpad, item_cap, nrb;
};

static int rows_per_wave_blocks(int rmax) { return rmax <= 64 ? 1 : (rmax <= 128 ? 2 : 4); }

static AttnLayout attn_layout(int B, int Hkv, int G, int HD, int max_pages, int max_draft, int kv_chunk) {
  AttnLayout L;
  const int rmax = G * (1 + max_draft);
  L.nrb = rows_per_wave_blocks(rmax);
  L.rpad = (rmax + 15) / 16 * 16;
  const long long max_keys = (long long)max_pages * kPage;
  long long cap;
  if (kv_chunk > 0) {
    cap = (long long)B * Hkv * ((max_keys + kv_chunk - 1) / kv_chunk);
  } else {
    // auto chunk = clamp(ceil(keys*Hkv/target), kMinChunk, kMaxChunk): below the upper clamp the
    // items number at most target + B*Hkv, at it at most B*Hkv*ceil(max_keys/kMaxChunk)
    cap = kTargetItems + (long long)B * Hkv;
    const long long by_max = (long long)B * Hkv * ((max_keys + kMaxChunk - 1) / kMaxChunk);
    cap = cap > by_max ? cap : by_max;
    const long long by_min = (long long)B * Hkv * ((max_keys + kMinChunk - 1) / kMinChunk);
    cap = cap < by_min ? cap : by_min;
  }
  if (cap < 1) cap = 1;
  L.item_cap = (int)cap;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.plan_off = take((size_t)(kPlanHeader + B + 1) * 4);
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

template <int HD, int NRB, int OUTF>
static void launch_main(const AttnParams& p, int grid, hipStream_t st) {
  verify_attn_main<HD, NRB, OUTF><<<grid, kThreads, 0, st>>>(p);
}

template <int HD, int OUTF>
static void launch_main_nrb(int nrb, const AttnParams& p, int grid, hipStream_t st) {
  if (nrb == 1) launch_main<HD, 1, OUTF>(p, grid, st);
  else if (nrb == 2) launch_main<HD, 2, OUTF>(p, grid, st);
  else launch_main<HD, 4, OUTF>(p, grid, st);
}

hipError_t sdv_attn_launch(const SdAttnLaunch& a) {
  const AttnLayout L = attn_layout(a.B, a.Hkv, a.G, a.head_dim, a.max_pages, a.max_draft, a.kv_chunk);
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

  int dev = 0, cus = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int per_cu = L.nrb >= 4 ? 1 : 2;
  const int grid = (int)std::min<long long>((long long)cus * per_cu, L.item_cap);

  verify_attn_plan<<<1, kThreads, 0, a.stream>>>(p, a.kv_chunk);
  if (a.head_dim == 128) {
    if (a.out_f32) launch_main_nrb<128, 1>(L.nrb, p, grid, a.stream);
    else launch_main_nrb<128, 0>(L.nrb, p, grid, a.stream);
  } else {
    if (a.out_f32) launch_main_nrb<64, 1>(L.nrb, p, grid, a.stream);
    else launch_main_nrb<64, 0>(L.nrb, p, grid, a.stream);
  }
  const int row_blocks = L.rpad / 8;
  const int cgrid = a.B * a.Hkv * row_blocks;
  if (a.head_dim == 128) {
    if (a.out_f32) verify_attn_combine<128, 1><<<cgrid, kThreads, 0, a.stream>>>(p);
    else verify_attn_combine<128, 0><<<cgrid, kThreads, 0, a.stream>>>(p);
  } else {
    if (a.out_f32) verify_attn_combine<64, 1><<<cgrid, kThreads, 0, a.stream>>>(p);
    else verify_attn_combine<64, 0><<<cgrid, kThreads, 0, a.stream>>>(p);
  }
  return hipGetLastError();
}
