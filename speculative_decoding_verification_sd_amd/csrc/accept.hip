// Accept / reject over the vocabulary on gfx950.
//
// The target walks the drafts left to right and keeps them until the first
// failure, then always adds one token of its own, so AL is in [1, 1+D]
// ("Co-Designing AI Models Using Speculative Decoding for Faster LLM
// Inference", section "What is speculative decoding?").  Greedy: a draft
// passes when it is the target's top token.  Stochastic: draft x passes with
// probability min(1, p(x)/q(x)); at the first failure the token is resampled
// from max(0, p - q) renormalised, which makes the output follow p exactly
// ("How does speculative decoding speed up LLM inference?", sections
// "Mechanism" and "Math intuition").
//
// Kernels (all vocab-parallel except the per-sequence decision):
//   1. accept_rowstats   grid = rows x vocab chunks.  Per chunk of 4096 logits:
//                        max, lowest-index argmax and sum of exp(x - max)
//                        (fp32 exp, fp64 accumulation).  One pass over every
//                        target (and draft) row: this is the step's HBM cost.
//   2. accept_decide     one workgroup per sequence.  Merges the chunk
//                        statistics into log-normalisers (fp64), runs the D_b
//                        tests in parallel (fp64 ratios), finds the first
//                        failure n, writes AL and the accepted tokens.
//   3. accept_residual   grid = vocab chunks x sequences (stochastic only).
//                        fp64 chunk sums of the residual max(0, p - q) at row
//                        n (or of p at row D when everything passed).
//   4. accept_sample     one workgroup per sequence.  Finds the chunk holding
//                        u*Z from the chunk sums, rebuilds that chunk's fp64
//                        weights and scans them to the first prefix sum > u*Z.

#include <math.h>
#include <limits.h>

#include "common.h"

namespace sdv {

constexpr int kAccThreads = 256;
constexpr int kChunk = 4096;                      // logits per workgroup
constexpr int kPerThread = kChunk / kAccThreads;  // 16

struct RowPart {
  float m;     // chunk max
  int idx;     // lowest index attaining it
  double s;    // sum of exp(x - m) over the chunk
};

struct SeqState {
  int n;            // leading passes
  int residual;     // 1: sample max(0, p - q) at row n; 0: sample p at row D
  double lse_p;     // log-normaliser of the target row n
  double lse_q;     // log-normaliser of the draft row n (residual only)
  double pad;
};

struct AccParams {
  const float* target;
  const float* draft;
  const int* tokens;
  const int* q_start;
  const float* uniforms;
  int* accept_len;
  int* out_tokens;
  RowPart* part;      // [rows, nchunk]
  SeqState* state;    // [B]
  double* rsum;       // [B, nchunk, 2]  (residual, p) chunk sums
  int B, T, V, nchunk, max_draft;
};

__device__ __forceinline__ bool better(float m1, int i1, float m0, int i0) {
  return m1 > m0 || (m1 == m0 && i1 < i0);
}

__device__ __forceinline__ void block_argmax(float& m, int& idx, float* sm, int* si) {
  for (int off = 32; off > 0; off >>= 1) {
    const float om = __shfl_xor(m, off);
    const int oi = __shfl_xor(idx, off);
    if (better(om, oi, m, idx)) { m = om; idx = oi; }
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[w] = m; si[w] = idx; }
  __syncthreads();
  m = sm[0];
  idx = si[0];
  for (int k = 1; k < kAccThreads / 64; ++k)
    if (better(sm[k], si[k], m, idx)) { m = sm[k]; idx = si[k]; }
  __syncthreads();
}

__device__ __forceinline__ double block_sum(double v, double* sd) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sd[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < kAccThreads / 64; ++k) t += sd[k];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int seq_d(const AccParams& p, int b) {
  return min(max(p.q_start[b + 1] - p.q_start[b] - 1, 0), p.max_draft);
}

// The sequence's target rows [t0, t0+D] and draft rows [d0, d0+D) lie inside the inputs.
__device__ __forceinline__ bool seq_ok(const AccParams& p, int t0, int D, int d0) {
  return t0 >= 0 && t0 + D < p.T && d0 >= 0 && d0 + D <= p.T - p.B;
}

// ---------------------------------------------------------------------------
template <int STOCH, int VEC4>
__global__ __launch_bounds__(kAccThreads) void accept_rowstats(AccParams p) {
  __shared__ float sm[4];
  __shared__ int si[4];
  __shared__ double sd[4];
  const int row = blockIdx.x / p.nchunk;
  const int c = blockIdx.x - row * p.nchunk;
  const float* src = row < p.T ? p.target + (size_t)row * p.V : p.draft + (size_t)(row - p.T) * p.V;
  const int tid = threadIdx.x;
  const int j0 = c * kChunk;

  float x[kPerThread];
  int jx[kPerThread];
  if (VEC4) {
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const int j = j0 + (k * kAccThreads + tid) * 4;
      f32x4 v;
      if (j + 3 < p.V) {
        v = *(const f32x4*)(src + j);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = j + e < p.V ? src[j + e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[k * 4 + e] = v[e]; jx[k * 4 + e] = j + e; }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int j = j0 + k * kAccThreads + tid;
      x[k] = j < p.V ? src[j] : -INFINITY;
      jx[k] = j;
    }
  }
  // indices visited in increasing order: strict '>' keeps the lowest index on ties
  float m = -INFINITY;
  int idx = INT_MAX;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    if (x[k] > m || (idx == INT_MAX && jx[k] < p.V && x[k] == m)) { m = x[k]; idx = jx[k]; }
  block_argmax(m, idx, sm, si);

  double s = 0.0;
  if (STOCH && m != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) s += (double)expf(x[k] - m);
    s = block_sum(s, sd);
  }
  if (tid == 0) {
    RowPart r;
    r.m = m;
    r.idx = idx;
    r.s = s;
    p.part[(size_t)row * p.nchunk + c] = r;
  }
}

// ---------------------------------------------------------------------------
template <int STOCH>
__global__ __launch_bounds__(kAccThreads) void accept_decide(AccParams p) {
  extern __shared__ double dyn[];               // lse_p[D+1], lse_q[D], argmax[D+1]
  __shared__ int first_fail;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  double* lse_p = dyn;
  double* lse_q = dyn + (p.max_draft + 1);
  int* amax = (int*)(dyn + 2 * p.max_draft + 1);
  const bool ok = seq_ok(p, t0, D, d0);
  if (!ok) {
    if (tid == 0) p.accept_len[b] = 0;
    return;
  }

  const int nrows = STOCH ? 2 * D + 1 : D + 1;
  for (int r = tid; r < nrows; r += kAccThreads) {
    const int prow = r <= D ? t0 + r : p.T + d0 + (r - D - 1);
    const RowPart* pr = p.part + (size_t)prow * p.nchunk;
    float M = -INFINITY;
    int ai = INT_MAX;
    for (int c = 0; c < p.nchunk; ++c)
      if (better(pr[c].m, pr[c].idx, M, ai)) { M = pr[c].m; ai = pr[c].idx; }
    double lse = 0.0;
    if (STOCH) {
      double Z = 0.0;
      for (int c = 0; c < p.nchunk; ++c)
        if (pr[c].m != -INFINITY) Z += exp((double)pr[c].m - (double)M) * pr[c].s;
      lse = (double)M + log(Z);
    }
    if (r <= D) { lse_p[r] = lse; amax[r] = ai; }
    else lse_q[r - D - 1] = lse;
  }
  if (tid == 0) first_fail = D;
  __syncthreads();

  for (int i = tid; i < D; i += kAccThreads) {
    const int x = p.tokens[d0 + i];
    bool pass = false;
    if (x >= 0 && x < p.V) {
      if (!STOCH) {
        pass = x == amax[i];
      } else {
        const double lp = (double)p.target[(size_t)(t0 + i) * p.V + x] - lse_p[i];
        const double lq = (double)p.draft[(size_t)(d0 + i) * p.V + x] - lse_q[i];
        const double r = exp(lp - lq);
        pass = (double)p.uniforms[t0 + i] < r;
      }
    }
    if (!pass) atomicMin(&first_fail, i);
  }
  __syncthreads();
  const int n = first_fail;
  for (int k = tid; k <= D; k += kAccThreads) {
    int tok = -1;
    if (k < n) tok = p.tokens[d0 + k];
    else if (k == n && !STOCH) tok = amax[n];
    p.out_tokens[t0 + k] = tok;
  }
  if (tid == 0) {
    p.accept_len[b] = n + 1;
    if (STOCH) {
      SeqState st;
      st.n = n;
      st.residual = n < D;
      st.lse_p = lse_p[n];
      st.lse_q = n < D ? lse_q[n] : 0.0;
      st.pad = 0.0;
      p.state[b] = st;
    }
  }
}

// fp64 weight of token j for the sampling row of one sequence.
__device__ __forceinline__ void sample_weights(const AccParams& p, const SeqState& st, int t0, int d0, int j,
                                               double& w, double& pj) {
  const double pt = exp((double)p.target[(size_t)(t0 + st.n) * p.V + j] - st.lse_p);
  pj = pt;
  if (st.residual) {
    const double qt = exp((double)p.draft[(size_t)(d0 + st.n) * p.V + j] - st.lse_q);
    w = fmax(0.0, pt - qt);
  } else {
    w = pt;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAccThreads) void accept_residual(AccParams p) {
  __shared__ double sd[4];
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int t0 = p.q_start[b];
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, seq_d(p, b), d0)) return;
  const SeqState st = p.state[b];
  double zw = 0.0, zp = 0.0;
#pragma unroll 4
  for (int k = 0; k < kPerThread; ++k) {
    const int j = c * kChunk + k * kAccThreads + threadIdx.x;
    if (j < p.V) {
      double w, pj;
      sample_weights(p, st, t0, d0, j, w, pj);
      zw += w;
      zp += pj;
    }
  }
  zw = block_sum(zw, sd);
  zp = block_sum(zp, sd);
  if (threadIdx.x == 0) {
    p.rsum[((size_t)b * p.nchunk + c) * 2 + 0] = zw;
    p.rsum[((size_t)b * p.nchunk + c) * 2 + 1] = zp;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAccThreads) void accept_sample(AccParams p) {
  __shared__ double scan[kAccThreads];
  __shared__ int s_chunk, s_usep, s_tok;
  __shared__ double s_base, s_T;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, D, d0)) return;
  SeqState st = p.state[b];

  if (tid == 0) {
    const double* rs = p.rsum + (size_t)b * p.nchunk * 2;
    double Z = 0.0;
    for (int c = 0; c < p.nchunk; ++c) Z += rs[2 * c];
    int usep = 0;
    if (!(Z > 0.0)) {
      usep = 1;
      Z = 0.0;
      for (int c = 0; c < p.nchunk; ++c) Z += rs[2 * c + 1];
    }
    const double T = (double)p.uniforms[t0 + D] * Z;
    double acc = 0.0;
    int cs = -1;
    for (int c = 0; c < p.nchunk; ++c) {
      const double nxt = acc + rs[2 * c + usep];
      if (nxt > T) { cs = c; break; }
      acc = nxt;
    }
    if (cs < 0) {                     // rounding: fall back to the last chunk with weight
      cs = 0;
      for (int c = 0; c < p.nchunk; ++c) if (rs[2 * c + usep] > 0.0) cs = c;
      acc = -INFINITY;                // never satisfied below -> last positive weight
    }
    s_chunk = cs;
    s_base = acc;
    s_T = T;
    s_usep = usep;
    s_tok = INT_MAX;
  }
  __syncthreads();
  if (s_usep) st.residual = 0;
  const int j0 = s_chunk * kChunk + tid * kPerThread;
  double w[kPerThread];
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int j = j0 + e;
    double pj;
    w[e] = 0.0;
    if (j < p.V) sample_weights(p, st, t0, d0, j, w[e], pj);
    tsum += w[e];
  }
  // inclusive scan of the per-thread sums (ascending token order)
  scan[tid] = tsum;
  __syncthreads();
  for (int off = 1; off < kAccThreads; off <<= 1) {
    const double add = tid >= off ? scan[tid - off] : 0.0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  double C = s_base + (scan[tid] - tsum);
  int cand = INT_MAX;
  int last_pos = -1;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    C += w[e];
    if (cand == INT_MAX && C > s_T) cand = j0 + e;
    if (w[e] > 0.0) last_pos = j0 + e;
  }
  if (cand != INT_MAX) atomicMin(&s_tok, cand);
  __syncthreads();
  if (s_tok == INT_MAX) {             // rounding left u*Z past this chunk's scan
    scan[tid] = (double)last_pos;
    __syncthreads();
    if (tid == 0) {
      int best = -1;
      for (int k = 0; k < kAccThreads; ++k) best = max(best, (int)scan[k]);
      s_tok = best < 0 ? s_chunk * kChunk : best;
    }
    __syncthreads();
  }
  if (tid == 0) p.out_tokens[t0 + st.n] = s_tok;
}

struct AccLayout {
  size_t part_off, state_off, rsum_off, total;
  int nchunk;
};

static AccLayout acc_layout(int B, int T, int V, int stochastic) {
  AccLayout L;
  L.nchunk = (V + kChunk - 1) / kChunk;
  const size_t rows = stochastic ? (size_t)T + (size_t)(T - B) : (size_t)T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.part_off = take(rows * L.nchunk * sizeof(RowPart));
  L.state_off = take((size_t)B * sizeof(SeqState));
  L.rsum_off = take((size_t)B * L.nchunk * 2 * sizeof(double));
  L.total = off;
  return L;
}

}  // namespace sdv

using namespace sdv;

size_t sdv_accept_workspace_bytes(int B, int T, int V, int stochastic) {
  return acc_layout(B, T, V, stochastic).total;
}

hipError_t sdv_accept_launch(const SdAccLaunch& a) {
  const AccLayout L = acc_layout(a.B, a.T, a.V, a.stochastic);
  unsigned char* ws = (unsigned char*)a.workspace;
  AccParams p;
  p.target = a.target;
  p.draft = a.draft;
  p.tokens = a.tokens;
  p.q_start = a.q_start;
  p.uniforms = a.uniforms;
  p.accept_len = a.accept_len;
  p.out_tokens = a.out_tokens;
  p.part = (RowPart*)(ws + L.part_off);
  p.state = (SeqState*)(ws + L.state_off);
  p.rsum = (double*)(ws + L.rsum_off);
  p.B = a.B;
  p.T = a.T;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.max_draft = a.max_draft;

  const bool vec4 = (a.V % 4 == 0) && ((uintptr_t)a.target % 16 == 0) &&
                    (!a.stochastic || (uintptr_t)a.draft % 16 == 0);
  const size_t rows = a.stochastic ? (size_t)a.T + (size_t)(a.T - a.B) : (size_t)a.T;
  const unsigned grid1 = (unsigned)(rows * L.nchunk);
  const size_t dyn = (size_t)(2 * a.max_draft + 1) * sizeof(double) + (size_t)(a.max_draft + 1) * sizeof(int);
  if (a.stochastic) {
    if (vec4) accept_rowstats<1, 1><<<grid1, kAccThreads, 0, a.stream>>>(p);
    else accept_rowstats<1, 0><<<grid1, kAccThreads, 0, a.stream>>>(p);
    accept_decide<1><<<a.B, kAccThreads, dyn, a.stream>>>(p);
    accept_residual<<<dim3(L.nchunk, a.B), kAccThreads, 0, a.stream>>>(p);
    accept_sample<<<a.B, kAccThreads, 0, a.stream>>>(p);
  } else {
    if (vec4) accept_rowstats<0, 1><<<grid1, kAccThreads, 0, a.stream>>>(p);
    else accept_rowstats<0, 0><<<grid1, kAccThreads, 0, a.stream>>>(p);
    accept_decide<0><<<a.B, kAccThreads, dyn, a.stream>>>(p);
  }
  return hipGetLastError();
}
