// Internal helpers shared by the gfx950 kernels of the verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace sdv

// Host-side launch entry points implemented in the kernel translation units.
struct SdAttnLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* kv_len;
  const int32_t* q_start;
  void* out;
  void* workspace;
  int B, Hkv, G, head_dim, max_pages, num_pages, max_draft, out_f32, kv_chunk, total_q;
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
  hipStream_t stream;
};

size_t sdv_attn_workspace_bytes(int B, int Hkv, int G, int head_dim, int max_pages, int max_draft,
                                int kv_chunk);
hipError_t sdv_attn_launch(const SdAttnLaunch& a);
size_t sdv_accept_workspace_bytes(int B, int T, int V, int stochastic);
hipError_t sdv_accept_launch(const SdAccLaunch& a);
