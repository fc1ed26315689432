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
// Kernels:
//   1. accept_rowstats   grid = rows x vocab chunks (8192 logits each).  Chunk
//                        max (greedy: lowest-index argmax; stochastic: sum of
//                        exp(x - max) accumulated in fp64).  One pass over every
//                        target (and draft) row: this is the step's HBM cost.
//   2. accept_decide     one workgroup per sequence.  Loads the sequence's
//                        chunk statistics into LDS, merges them into per-row
//                        log-normalisers (fp64), runs the D_b tests in parallel
//                        (fp64 ratios), finds the first failure n, writes AL
//                        and the accepted tokens, and (stochastic) resets the
//                        sequence's arrival counter for kernel 3.
//   3. accept_sample     grid = vocab chunks x sequences (stochastic only).
//                        fp64 chunk sums of the residual max(0, p - q) at row
//                        n (of p at row D when every draft passed); the last
//                        chunk of a sequence to finish then finds the chunk
//                        holding u*Z and scans it in fp64 to the first prefix
//                        sum > u*Z.

#include <limits.h>
#include <math.h>

#include "common.h"

namespace sdv {

constexpr int kAccThreads = 256;
constexpr int kChunk = 8192;                      // logits per row-statistics workgroup
constexpr int kPerThread = kChunk / kAccThreads;  // 32
constexpr int kSChunk = 4096;                     // logits per sampling workgroup
constexpr int kSPerThread = kSChunk / kAccThreads;
constexpr int kDecideSlots = 2048;                // chunk statistics staged in LDS per pass

struct RowPart {
  float m;     // chunk max
  int idx;     // lowest index attaining it (greedy)
  double s;    // sum of exp(x - m) over the chunk (stochastic)
};

struct SeqState {
  int n;            // leading passes
  int residual;     // 1: sample max(0, p - q) at row n; 0: sample p at row D
  double lse_p;     // log-normaliser of the target row n
  double lse_q;     // log-normaliser of the draft row n (residual only)
  unsigned arrived; // sampling workgroups done (reset by accept_decide)
  int pad;
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
  double* rsum;       // [B, nschunk, 2]  (residual, p) chunk sums
  int B, T, V, nchunk, nschunk, max_draft;
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

__device__ __forceinline__ float block_max(float m, float* sm) {
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm[w] = m;
  __syncthreads();
  m = sm[0];
  for (int k = 1; k < kAccThreads / 64; ++k) m = fmaxf(m, sm[k]);
  __syncthreads();
  return m;
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

  // element k of this thread has index j0 + (k/4)*1024 + tid*4 + k%4 (VEC4) or
  // j0 + k*256 + tid (scalar): increasing in k either way
  float x[kPerThread];
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
      for (int e = 0; e < 4; ++e) x[k * 4 + e] = v[e];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int j = j0 + k * kAccThreads + tid;
      x[k] = j < p.V ? src[j] : -INFINITY;
    }
  }
  auto index_of = [&](int k) {
    return VEC4 ? j0 + ((k >> 2) * kAccThreads + tid) * 4 + (k & 3) : j0 + k * kAccThreads + tid;
  };

  if (!STOCH) {
    // lowest-index maximum: strict '>' over increasing indices; a row of -inf
    // still reports a real index (first element inside the vocabulary)
    float m = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int j = index_of(k);
      if (x[k] > m || (idx == INT_MAX && j < p.V)) { m = x[k]; idx = j; }
    }
    block_argmax(m, idx, sm, si);
    if (tid == 0) {
      RowPart r;
      r.m = m;
      r.idx = idx;
      r.s = 0.0;
      p.part[(size_t)row * p.nchunk + c] = r;
    }
  } else {
    float m = x[0];
#pragma unroll
    for (int k = 1; k < kPerThread; ++k) m = fmaxf(m, x[k]);
    m = block_max(m, sm);
    double s = 0.0;
    if (m != -INFINITY) {
      // exp(x - m) as 2^((x - m) log2 e); fp32 terms, fp64 running sum
      const float ml = m * 1.4426950408889634f;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) s += (double)fast_exp2(fmaf(x[k], 1.4426950408889634f, -ml));
      s = block_sum(s, sd);
    }
    if (tid == 0) {
      RowPart r;
      r.m = m;
      r.idx = 0;
      r.s = s;
      p.part[(size_t)row * p.nchunk + c] = r;
    }
  }
}

// ---------------------------------------------------------------------------
template <int STOCH>
__global__ __launch_bounds__(kAccThreads) void accept_decide(AccParams p) {
  extern __shared__ double dyn[];               // lse_p[D+1], lse_q[D], argmax[D+1]
  __shared__ RowPart stage[kDecideSlots];
  __shared__ int first_fail;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  double* lse_p = dyn;
  double* lse_q = dyn + (p.max_draft + 1);
  int* amax = (int*)(dyn + 2 * p.max_draft + 1);
  if (!seq_ok(p, t0, D, d0)) {
    if (tid == 0) p.accept_len[b] = 0;
    return;
  }

  // rows: r <= D -> target row t0+r; r > D -> draft row d0+r-D-1
  const int nrows = STOCH ? 2 * D + 1 : D + 1;
  const int rows_per_pass = max(1, kDecideSlots / p.nchunk);
  for (int r0 = 0; r0 < nrows; r0 += rows_per_pass) {
    const int nr = min(rows_per_pass, nrows - r0);
    __syncthreads();
    for (int e = tid; e < nr * p.nchunk; e += kAccThreads) {
      const int r = r0 + e / p.nchunk;
      const int prow = r <= D ? t0 + r : p.T + d0 + (r - D - 1);
      stage[e] = p.part[(size_t)prow * p.nchunk + (e % p.nchunk)];
    }
    __syncthreads();
    for (int rr = tid; rr < nr; rr += kAccThreads) {
      const RowPart* pr = stage + rr * p.nchunk;
      const int r = r0 + rr;
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
      st.arrived = 0u;
      st.pad = 0;
      p.state[b] = st;
    }
  }
}

// fp64 weights of token j for the sampling row of one sequence.
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
__global__ __launch_bounds__(kAccThreads) void accept_sample(AccParams p) {
  __shared__ double sd[4];
  __shared__ double scan[kAccThreads];
  __shared__ int s_last, s_chunk, s_usep, s_tok;
  __shared__ double s_base, s_T;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, D, d0)) return;
  SeqState st = p.state[b];

  // (1) this chunk's fp64 sums of the residual (or p) and of p
  double zw = 0.0, zp = 0.0;
#pragma unroll 4
  for (int k = 0; k < kSPerThread; ++k) {
    const int j = c * kSChunk + k * kAccThreads + tid;
    if (j < p.V) {
      double w, pj;
      sample_weights(p, st, t0, d0, j, w, pj);
      zw += w;
      zp += pj;
    }
  }
  zw = block_sum(zw, sd);
  zp = block_sum(zp, sd);
  if (tid == 0) {
    // Hand-off between workgroups of one sequence, possibly on different XCDs
    // (separate L2s): the sums are agent-scope atomic stores, which are
    // coherent across XCDs, and complete (vmcnt 0) before the arrival count.
    // A release fence would do the same by writing back the whole L2.
    double* dst = p.rsum + ((size_t)b * p.nschunk + c) * 2;
    __hip_atomic_store(dst, zw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 1, zp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const unsigned prev = __hip_atomic_fetch_add(&p.state[b].arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(p.nschunk - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // (2) last chunk to finish: find the chunk holding u*Z, then scan it.  The
  // chunk sums are read once each, in parallel, and scanned in LDS.
  double* rsb = p.rsum + (size_t)b * p.nschunk * 2;
  auto rs_at = [&](int i) { return __hip_atomic_load(rsb + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  zw = 0.0;
  zp = 0.0;
  for (int k = tid; k < p.nschunk; k += kAccThreads) {
    zw += rs_at(2 * k);
    zp += rs_at(2 * k + 1);
  }
  zw = block_sum(zw, sd);
  zp = block_sum(zp, sd);
  const int usep = !(zw > 0.0);                   // the residual has no mass: sample p
  const double T = (double)p.uniforms[t0 + D] * (usep ? zp : zw);
  if (tid == 0) {
    s_chunk = INT_MAX;
    s_tok = -1;                                   // last chunk with weight (rounding fallback)
  }
  double carry = 0.0;
  for (int base = 0; base < p.nschunk; base += kAccThreads) {
    const int k = base + tid;
    const double v = k < p.nschunk ? rs_at(2 * k + usep) : 0.0;
    scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kAccThreads; off <<= 1) {
      const double add = tid >= off ? scan[tid - off] : 0.0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const double incl = carry + scan[tid];
    if (k < p.nschunk && incl > T) atomicMin(&s_chunk, k);
    if (v > 0.0) atomicMax(&s_tok, k);
    __syncthreads();
    if (k == s_chunk) s_base = incl - v;
    carry += scan[kAccThreads - 1];
    __syncthreads();
    if (s_chunk != INT_MAX) break;
  }
  if (tid == 0) {
    if (s_chunk == INT_MAX) {                     // prefix never passed u*Z
      s_chunk = max(s_tok, 0);
      s_base = -INFINITY;                         // never satisfied below -> last positive weight
    }
    s_T = T;
    s_usep = usep;
    s_tok = INT_MAX;
  }
  __syncthreads();
  if (s_usep) st.residual = 0;
  const int j0 = s_chunk * kSChunk + tid * kSPerThread;
  double w[kSPerThread];
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < kSPerThread; ++e) {
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
  for (int e = 0; e < kSPerThread; ++e) {
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
      s_tok = best < 0 ? s_chunk * kSChunk : best;
    }
    __syncthreads();
  }
  if (tid == 0) p.out_tokens[t0 + st.n] = s_tok;
}

struct AccLayout {
  size_t part_off, state_off, rsum_off, total;
  int nchunk, nschunk;
};

static AccLayout acc_layout(int B, int T, int V, int stochastic) {
  AccLayout L;
  L.nchunk = (V + kChunk - 1) / kChunk;
  L.nschunk = (V + kSChunk - 1) / kSChunk;
  const size_t rows = stochastic ? (size_t)T + (size_t)(T - B) : (size_t)T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.part_off = take(rows * L.nchunk * sizeof(RowPart));
  L.state_off = take((size_t)B * sizeof(SeqState));
  L.rsum_off = take((size_t)B * L.nschunk * 2 * sizeof(double));
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
  p.nschunk = L.nschunk;
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
    accept_sample<<<dim3(L.nschunk, a.B), kAccThreads, 0, a.stream>>>(p);
  } else {
    if (vec4) accept_rowstats<0, 1><<<grid1, kAccThreads, 0, a.stream>>>(p);
    else accept_rowstats<0, 0><<<grid1, kAccThreads, 0, a.stream>>>(p);
    accept_decide<0><<<a.B, kAccThreads, dyn, a.stream>>>(p);
  }
  return hipGetLastError();
}
