// Opt-in check of the device-side input contract of the verify step, on
// gfx950.  The verify kernels themselves only clamp what they index (so that
// bad inputs cannot fault); this pass reports which part of the contract the
// inputs break, as bits of one status word:
//   SD_BAD_Q_START  q_start[0] != 0, a sequence with no row or more than
//                   1+max_draft rows, or q_start[B] != total_q
//   SD_BAD_KV_LEN   kv_len[b] below the sequence's 1+D_b block, or above
//                   max_pages*16 keys
//   SD_BAD_PAGE     a page id among a sequence's first ceil(kv_len/16)
//                   block-table entries outside [0, num_pages)
//   SD_BAD_TOKEN    a drafted token outside [0, V)
//   SD_BAD_UNIFORM  a uniform outside [0, 1) (NaN included)
//   SD_BAD_LOGITS   a NaN or +inf logit, or a row whose logits are all -inf
// Every index is range-checked before it is read, whatever the other inputs
// hold, so the pass itself stays in bounds on any input.

#include "common.h"
#include "sd_verify.h"

namespace sdv {

constexpr int kValThreads = 256;

__global__ void validate_clear(uint32_t* status) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *status = 0u;
}

// One workgroup per sequence.
__global__ __launch_bounds__(kValThreads) void validate_seqs(SdValidateLaunch v) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int t0 = v.q_start[b], t1 = v.q_start[b + 1];
  const bool q_ok = t0 >= 0 && t1 > t0 && t1 <= v.T && t1 - t0 <= 1 + v.max_draft && (b > 0 || t0 == 0) &&
                    (b < v.B - 1 || t1 == v.T);
  const int D = q_ok ? t1 - t0 - 1 : 0;
  uint32_t bad = 0u;
  if (tid == 0 && !q_ok) bad |= SD_BAD_Q_START;
  if (v.kv_len) {
    const int n = v.kv_len[b];
    const long long max_keys = (long long)v.max_pages * 16;
    if (tid == 0 && (n < 0 || n > max_keys || (q_ok && n < 1 + D))) bad |= SD_BAD_KV_LEN;
    const int npages = (int)((min((long long)max(n, 0), max_keys) + 15) / 16);
    const int* row = v.block_table + (size_t)b * v.max_pages;
    for (int j = tid; j < npages; j += kValThreads) {
      const int pid = row[j];
      if (pid < 0 || pid >= v.num_pages) bad |= SD_BAD_PAGE;
    }
  }
  if (q_ok) {
    // the sequence's drafted tokens sit at (t0 - b) + i, i < D, inside [0, T - B)
    const int d0 = t0 - b;
    for (int i = tid; i < D; i += kValThreads) {
      if (d0 + i < 0 || d0 + i >= v.T - v.B) {
        bad |= SD_BAD_Q_START;          // the blocks of earlier sequences are inconsistent
      } else if (v.tokens) {
        const int x = v.tokens[d0 + i];
        if (x < 0 || x >= v.V) bad |= SD_BAD_TOKEN;
      }
    }
    if (v.uniforms)
      for (int i = tid; i <= D; i += kValThreads) {
        const float u = v.uniforms[t0 + i];
        if (!(u >= 0.f && u < 1.f)) bad |= SD_BAD_UNIFORM;
      }
  }
  // one atomic per wave that found something
  const unsigned long long any = __ballot(bad != 0u);
  if (any) {
    uint32_t w = bad;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) w |= (uint32_t)__shfl_xor((int)w, off);
    if ((tid & 63) == 0) atomicOr(v.status, w);
  }
}

// One workgroup per logit row: the target rows (rows_t of them), then the draft rows.
__global__ __launch_bounds__(kValThreads) void validate_logits(SdValidateLaunch v, int rows_t, int rows) {
  const int r = blockIdx.x;
  if (r >= rows) return;
  const float* row = r < rows_t ? v.target + (size_t)r * v.V : v.draft + (size_t)(r - rows_t) * v.V;
  bool nan_or_pinf = false, any_above = false;
  for (int j = threadIdx.x; j < v.V; j += kValThreads) {
    const float x = row[j];
    if (x != x || x == INFINITY) nan_or_pinf = true;
    if (x > -INFINITY) any_above = true;
  }
  const bool bad_elem = __syncthreads_or(nan_or_pinf);
  const bool finite_row = __syncthreads_or(any_above);
  if (threadIdx.x == 0 && (bad_elem || !finite_row)) atomicOr(v.status, (uint32_t)SD_BAD_LOGITS);
}

}  // namespace sdv

using namespace sdv;

hipError_t sdv_validate_launch(const SdValidateLaunch& v) {
  validate_clear<<<1, 64, 0, v.stream>>>(v.status);
  if (v.B > 0) validate_seqs<<<v.B, kValThreads, 0, v.stream>>>(v);
  const int rows_t = v.target ? v.T : 0;
  const int rows = rows_t + (v.draft ? v.T - v.B : 0);
  if (rows > 0) validate_logits<<<rows, kValThreads, 0, v.stream>>>(v, rows_t, rows);
  return hipGetLastError();
}
