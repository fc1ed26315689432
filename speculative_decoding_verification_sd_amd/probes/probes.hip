// Measurement kernels for bench.py (not part of the verify step): the MFMA
// throughput one wave per SIMD and two per SIMD reach on this GPU, and the SIMD
// each wave of an 8-wave workgroup runs on.  Built into libsdprobe.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// SIMD id of the calling wave: bits 5:4 of the HW_ID hardware register
// (s_getreg_b32 with hwreg(HW_REG_HW_ID, 4, 2)).
__device__ __forceinline__ int simd_id() {
  return (int)__builtin_amdgcn_s_getreg((4) | (4 << 6) | ((2 - 1) << 11));
}

// CU id of the calling wave: bits 11:8 of HW_ID.
__device__ __forceinline__ int cu_id() {
  return (int)__builtin_amdgcn_s_getreg((4) | (8 << 6) | ((4 - 1) << 11));
}

// One workgroup of 8 waves per CU (the LDS request keeps a second one out),
// as the verify-attention kernel runs: out[block*8 + wave] = SIMD id | CU id << 4.
__global__ __launch_bounds__(512, 1) void probe_wave_layout(int* out, int nblocks) {
  __shared__ int pad[32768];                 // 128 KiB
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) pad[blockIdx.x & 32767] = blockIdx.x;
  __syncthreads();
  if ((threadIdx.x & 63) == 0 && blockIdx.x < nblocks)
    out[blockIdx.x * 8 + wave] = simd_id() | (cu_id() << 4) | ((pad[blockIdx.x & 32767] == (int)blockIdx.x) << 12);
}

// MFMA issue rate: each wave runs `iters` rounds of CHAINS independent
// accumulation chains of v_mfma_f32_32x32x16_bf16 (or 16x16x32) from registers,
// and writes its accumulators so that nothing is dropped.  s_memtime brackets
// the loop (shader clock cycles) for the per-wave cycle count.
template <int SHAPE, int CHAINS>
__global__ __launch_bounds__(256) void probe_mfma(float* out, long long* cycles, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + e) & 7));
  }
  const long long t0 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
  if constexpr (SHAPE == 32) {
    f32x16 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[c][e];
  } else {
    f32x4 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += acc[c][e];
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

// MFMA / VALU co-execution: each round issues 4 independent 32x32x16 bf16
// MFMA chains and, after each MFMA, NV independent vector operations of kind
// KIND (1: v_exp_f32, 2: v_fma_f32) on their own data (NV = 0: MFMAs only;
// MFMA = false: the vector work alone).  If the SIMD overlaps the two kinds,
// the round takes the longer of the two; if not, their sum.
template <bool MFMA, int KIND, int NV>
__global__ __launch_bounds__(256) void probe_coexec(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  float v[4][NV > 0 ? NV : 1];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int k = 0; k < (NV > 0 ? NV : 1); ++k) v[c][k] = 1e-6f * (float)(threadIdx.x + 7 * k + c);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (MFMA) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if constexpr (KIND == 1) v[c][k] = __builtin_amdgcn_exp2f(v[c][k]) * -0.5f;
        else v[c][k] = fmaf(v[c][k], 0.999f, 1e-7f);
      }
    }
    if constexpr (MFMA && NV > 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, KIND == 1 ? 2 * NV : NV, 0);
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
#pragma unroll
    for (int k = 0; k < (NV > 0 ? NV : 1); ++k) sum += v[c][k];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

#define SDP_EXPORT extern "C" __attribute__((visibility("default")))

// nblocks workgroups; out int32 [nblocks * 8] (device).
SDP_EXPORT int sdp_wave_layout(int* out, int nblocks, void* stream) {
  if (!out || nblocks < 1) return 1;
  probe_wave_layout<<<nblocks, 512, 0, (hipStream_t)stream>>>(out, nblocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// shape 32 (32x32x16) or 16 (16x16x32); waves_per_simd 1 or 2 (workgroups of
// 256 threads, one or two per CU by the grid); out fp32 [grid * 256],
// cycles int64 [grid] (device).
SDP_EXPORT int sdp_mfma_peak(int shape, int grid, int iters, float* out, long long* cycles, void* stream) {
  if (!out || !cycles || grid < 1 || iters < 1) return 1;
  hipStream_t st = (hipStream_t)stream;
  if (shape == 32) probe_mfma<32, 4><<<grid, 256, 0, st>>>(out, cycles, iters);
  else if (shape == 16) probe_mfma<16, 8><<<grid, 256, 0, st>>>(out, cycles, iters);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// variant: 0 MFMA only; 1 MFMA + 2 exp per MFMA; 2 exp only (2 per slot);
// 3 MFMA + 8 fma per MFMA; 4 fma only (8 per slot).  out fp32 [grid * 256].
SDP_EXPORT int sdp_coexec(int variant, int grid, int iters, float* out, void* stream) {
  if (!out || grid < 1 || iters < 1) return 1;
  hipStream_t st = (hipStream_t)stream;
  switch (variant) {
    case 0: probe_coexec<true, 1, 0><<<grid, 256, 0, st>>>(out, iters); break;
    case 1: probe_coexec<true, 1, 2><<<grid, 256, 0, st>>>(out, iters); break;
    case 2: probe_coexec<false, 1, 2><<<grid, 256, 0, st>>>(out, iters); break;
    case 3: probe_coexec<true, 2, 8><<<grid, 256, 0, st>>>(out, iters); break;
    case 4: probe_coexec<false, 2, 8><<<grid, 256, 0, st>>>(out, iters); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
