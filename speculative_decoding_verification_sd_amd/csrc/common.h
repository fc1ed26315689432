// Internal helpers shared by the gfx950 kernels of the verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace sdv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

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

// A bare workgroup barrier.  s_barrier does not wait for this wave's own LDS
// stores (nor for its vector loads): the LDS-DMA ring uses it as is, because
// each wave waits for its DMA loads with s_waitcnt vmcnt before the barrier
// and writes no LDS with ordinary stores there.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A barrier that publishes this wave's LDS stores to the workgroup: wait until
// they have completed, then s_barrier.  Every hand-off of values through LDS
// by ordinary stores (a work index, partial results) goes through this.
__device__ __forceinline__ void block_sync_lds() {
  wait_lds();
  block_sync();
}

// One 16-byte-per-lane global->LDS DMA (global_load_lds_dwordx4, scalar-base
// form): lane i reads base + voff_i and its 16 bytes land at LDS byte address
// lds_addr + 16*i; base and lds_addr are wave-uniform (lds_addr goes to M0).
// Issued as inline asm so that the compiler's waitcount logic does not pace
// every later LDS read on these loads (it cannot tell ring stages apart and
// would wait for all of them); the ring waits for them explicitly with
// s_waitcnt vmcnt before its barrier.  The asm saves M0 in a scratch SGPR,
// sets it, issues the load (one wait state after the M0 write) and puts the
// saved value back, so M0 is unchanged across the statement and the compiler
// may keep anything of its own there.
// STREAM: data read once per call (the KV cache) goes with the non-temporal
// hint, so that it does not displace what the caches hold for reuse.
template <bool STREAM = false>
__device__ __forceinline__ void dma16(const unsigned char* base, unsigned voff, unsigned lds_addr) {
  // readfirstlane returns int: go through unsigned so the low word is zero-extended
  const uint64_t b = (uint64_t)base;
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  unsigned saved;
  if constexpr (STREAM)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3 nt\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sb)
                 : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sb)
                 : "memory");
}

}  // namespace sdv

// Host-side launch entry points implemented in the kernel translation units.
struct SdAttnLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* kv_len;
  const int32_t* q_start;
  const int32_t* parents;   // NULL: causal verify block; else draft-tree parents (see sd_verify_tree_attention)
  void* out;
  void* workspace;
  int B, Hkv, G, head_dim, max_pages, num_pages, max_draft, out_f32, kv_chunk, total_q;
  int v_key_major;          // 1: v_cache [P, H_kv, page, d] (like K); 0: [P, H_kv, d, page]
  float softmax_scale;
  hipStream_t stream;
};

struct SdAccLaunch {
  const float* target;
  const float* draft;
  const int32_t* tokens;
  const int32_t* q_start;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* out_tokens;
  void* workspace;
  int B, T, V, max_draft, stochastic;
  int lossy;              // relaxed acceptance: a draft also passes when its rows' JS distance <= js_threshold
  float js_threshold;
  float* out_entropy;     // [T-B] or NULL (relaxed only)
  float* out_js;          // [T-B] or NULL (relaxed only)
  hipStream_t stream;
};

size_t sdv_attn_workspace_bytes(int B, int Hkv, int G, int head_dim, int max_pages, int max_draft,
                                int kv_chunk);
hipError_t sdv_attn_launch(const SdAttnLaunch& a);
size_t sdv_accept_workspace_bytes(int B, int T, int V, int stochastic, int lossy);
// Library-held scratch of the no-allocation accept call (noalloc.hip).
size_t sdv_noalloc_scratch_bytes();
hipError_t sdv_noalloc_scratch(void** out);
hipError_t sdv_accept_launch(const SdAccLaunch& a);
hipError_t sdv_tree_accept_launch(const SdAccLaunch& a, const int32_t* parents, int32_t* out_nodes);

// A closed speculative-decoding loop on a bigram toy LM (loop.hip).
struct SdLoopLaunch {
  const float* W;         // [V, V] bigram logits (device)
  int32_t* hist;          // [B, max_len] histories (device, updated)
  int32_t* len;           // [B] lengths (device, updated)
  int32_t* al_trace;      // [steps, B] appended tokens per round (host)
  int32_t* tier_trace;    // [steps] draft length of each round (host)
  const int32_t* tiers;   // [ntiers] ascending draft lengths (host)
  void* workspace;
  int B, V, max_len, ngram, ntiers, steps, use_graphs;
  float ema_weight;
  hipStream_t stream;
};
size_t sdv_loop_workspace_bytes(int B, int V, int ntiers, int dmax);
hipError_t sdv_closed_loop(const SdLoopLaunch& c);

// Opt-in check of the inputs' device-side contract (validate.hip).  NULL
// pointers switch the matching checks off; status gets SD_BAD_* bits.
struct SdValidateLaunch {
  const int32_t* block_table;   // [B, max_pages] (NULL: no cache checks)
  const int32_t* kv_len;        // [B]
  const int32_t* q_start;       // [B+1]
  const int32_t* tokens;        // [T - B] drafted tokens (NULL: not checked)
  const float* uniforms;        // [T] (NULL: not checked)
  const float* target;          // [T, V] (NULL: not checked)
  const float* draft;           // [T - B, V] (NULL: not checked)
  uint32_t* status;             // one word, cleared then OR-ed
  int B, T, V, max_draft, max_pages, num_pages;
  hipStream_t stream;
};
hipError_t sdv_validate_launch(const SdValidateLaunch& v);

struct SdGemmLaunch {
  const void* x;
  const void* w;
  void* y;
  void* workspace;
  size_t workspace_bytes;
  int m, n, k;
  hipStream_t stream;
};

size_t sdv_gemm_workspace_bytes(int m, int n, int k);
hipError_t sdv_gemm_launch(const SdGemmLaunch& a);
