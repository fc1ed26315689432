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
//   2a. accept_decide    greedy: one workgroup per sequence merges the chunk
//                        argmaxes of its 1+D rows, compares the drafts, and
//                        writes AL, the accepted tokens and the correction.
//   2b. accept_finish    stochastic: grid = vocab chunks x sequences.  Every
//                        workgroup takes the sequence's decision itself (fp64
//                        log-normalisers merged from the chunk statistics, the
//                        D tests in fp64, the first failure n); workgroup 0
//                        writes AL, the accepted tokens and the decision.  Each
//                        workgroup then sums its chunk of the residual
//                        max(0, p - q) at row n (of p at row D when every
//                        draft passed) in fp64, per thread (16 consecutive
//                        tokens) and per chunk.
//   2c. accept_draw      stochastic: one workgroup per sequence finds the first
//                        prefix sum > u*Z by chunk, then 16-token slice, then
//                        token.  The kernel boundary orders the sums before
//                        their reads (no hand-off between workgroups).

#include <limits.h>
#include <algorithm>
#include <math.h>

#include "common.h"

namespace sdv {

constexpr int kAccThreads = 256;
// logits per row-statistics workgroup (build-time tunable)
#ifndef SDV_ACC_CHUNK
#define SDV_ACC_CHUNK 8192
#endif
constexpr int kChunk = SDV_ACC_CHUNK;
constexpr int kPerThread = kChunk / kAccThreads;  // 32 at the default chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSChunk = 4096;                     // logits per sampling workgroup
constexpr int kSPerThread = kSChunk / kAccThreads;  // 16: one slice of the sampling search per thread
static_assert(kSPerThread % 4 == 0 && kSPerThread <= 64, "a slice is scanned by one wave");
constexpr int kDecideSlots = 2048;
#ifndef SDV_ROWSTATS_WGS
#define SDV_ROWSTATS_WGS 1024
#endif
constexpr int kRowstatsWGs = SDV_ROWSTATS_WGS;     // accept_rowstats workgroups (persistent grid)
constexpr int kFinishWGs = 1024;                  // accept_finish workgroups in flight at once (4 per CU)

struct RowPart {
  float m;     // chunk max
  int idx;     // lowest index attaining it (greedy)
  double s;    // sum of exp(x - m) over the chunk (stochastic)
};

// The decision a sampling workgroup works from.
struct SeqState {
  int n;            // leading passes
  int residual;     // 1: sample max(0, p - q) at row n; 0: sample p at row D
  double lse_p;     // log-normaliser of the target row n
  double lse_q;     // log-normaliser of the draft row n (residual only)
};

struct SeqRec {      // a sequence's decision, from accept_finish to accept_draw
  double lse_p, lse_q;
  int n;
  float u;           // the sampling uniform u[t0 + D]
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
  SeqRec* seqrec;     // [B] decisions of the stochastic sequences
  double* rsum;       // [B, nschunk, 2]  (residual, p) chunk sums
  double* rsub;       // [B, nschunk, 256, 2]  (residual, p) sums of each thread's 16 tokens
  // relaxed acceptance only
  double* ent;        // [T-B, nchunk]  chunk sums of exp(x - m) (x - m) of the draft rows
  double* jsp;        // [T-B, nchunk]  chunk sums of the Jensen-Shannon terms
  float* out_ent;     // [T-B] draft entropy per drafted row (or NULL)
  float* out_js;      // [T-B] JS distance per drafted row (or NULL)
  float tau;          // JS threshold (< 0: off)
  int B, T, V, nchunk, nschunk, max_draft, vec4;
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

// Element k of this thread in a chunk of kChunk logits starting at j0: index
// j0 + (k/4)*1024 + tid*4 + k%4 (VEC4) or j0 + k*256 + tid (scalar),
// increasing in k either way; past the vocabulary it reads -inf.
template <int VEC4>
__device__ __forceinline__ int chunk_index(int j0, int k) {
  const int tid = threadIdx.x;
  return VEC4 ? j0 + ((k >> 2) * kAccThreads + tid) * 4 + (k & 3) : j0 + k * kAccThreads + tid;
}

template <int VEC4>
__device__ __forceinline__ void load_chunk(const float* src, int j0, int V, float (&x)[kPerThread]) {
  const int tid = threadIdx.x;
  if (VEC4) {
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const int j = j0 + (k * kAccThreads + tid) * 4;
      f32x4 v;
      if (j + 3 < V) {
        v = __builtin_nontemporal_load((const f32x4*)(src + j));   // streamed once: no cache residency
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = j + e < V ? src[j + e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[k * 4 + e] = v[e];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int j = j0 + k * kAccThreads + tid;
      x[k] = j < V ? src[j] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// MODE 0: greedy (lowest-index maximum); 1: stochastic (maximum and sum of
// exp(x - max)); 2: relaxed greedy acceptance (all of those, and for draft rows
// the sum of exp(x - max) (x - max), from which the row's entropy follows);
// 3: relaxed stochastic acceptance (as 2 without the argmax, which only the
// greedy test reads).
// Chunk g of the rows x chunks grid: row g / nchunk, chunk g % nchunk, whose
// logits the caller has loaded into x.
template <int MODE, int VEC4>
__device__ __forceinline__ void rowstats_chunk(const AccParams& p, int g, const float (&x)[kPerThread], float* sm,
                                               int* si, double* sd) {
  const int row = g / p.nchunk;
  const int c = g - row * p.nchunk;
  const int tid = threadIdx.x;
  const int j0 = c * kChunk;
  RowPart r;
  r.idx = 0;
  r.s = 0.0;
  float m;
  if (MODE == 0 || MODE == 2) {
    // lowest-index maximum: strict '>' over increasing indices; a row of -inf
    // still reports a real index (first element inside the vocabulary)
    m = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int j = chunk_index<VEC4>(j0, k);
      if (x[k] > m || (idx == INT_MAX && j < p.V)) { m = x[k]; idx = j; }
    }
    block_argmax(m, idx, sm, si);
    r.idx = idx;
  } else {
    m = x[0];
#pragma unroll
    for (int k = 1; k < kPerThread; ++k) m = fmaxf(m, x[k]);
    m = block_max(m, sm);
  }
  r.m = m;
  if (MODE != 0) {
    const bool ent = MODE >= 2 && row >= p.T;   // (uniform over the workgroup)
    double s = 0.0, s1 = 0.0;
    if (m != -INFINITY) {
      // exp(x - m) as 2^((x - m) log2 e): fp32 terms, fp64 running sums, the
      // terms summed eight at a time first (MODE 2, whose argmax holds more
      // registers: one at a time)
      const float ml = m * 1.4426950408889634f;
      if constexpr (MODE == 2) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
          const float e = fast_exp2(fmaf(x[k], 1.4426950408889634f, -ml));
          s += (double)e;
          if (ent && e > 0.f) s1 += (double)(e * (x[k] - m));
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < kPerThread; k0 += 8) {
          float a = 0.f, a1 = 0.f;
#pragma unroll
          for (int k = k0; k < k0 + 8; ++k) {
            const float e = fast_exp2(fmaf(x[k], 1.4426950408889634f, -ml));
            a += e;
            if (ent) a1 += e > 0.f ? e * (x[k] - m) : 0.f;
          }
          s += (double)a;
          if (ent) s1 += (double)a1;
        }
      }
      s = block_sum(s, sd);
      if (ent) s1 = block_sum(s1, sd);
    }
    r.s = s;
    if (ent && tid == 0) p.ent[(size_t)(row - p.T) * p.nchunk + c] = s1;
  }
  if (tid == 0) p.part[(size_t)row * p.nchunk + c] = r;
}

template <int VEC4>
__device__ __forceinline__ void rowstats_load(const AccParams& p, int g, float (&x)[kPerThread]) {
  const int row = g / p.nchunk;
  const int c = g - row * p.nchunk;
  const float* src = row < p.T ? p.target + (size_t)row * p.V : p.draft + (size_t)(row - p.T) * p.V;
  load_chunk<VEC4>(src, c * kChunk, p.V, x);
}

// A persistent grid over the rows x chunks: each workgroup takes chunks
// blockIdx.x, + gridDim.x, ..., and loads the next one before it reduces the
// current one, so that its loads stay in flight through the reductions.  Four
// waves per SIMD (at most 128 VGPRs) keep every workgroup of the grid resident.
template <int MODE, int VEC4>
__global__ __launch_bounds__(kAccThreads, 4) void accept_rowstats(AccParams p, int total) {
  __shared__ float sm[4];
  __shared__ int si[4];
  __shared__ double sd[4];
  float xa[kPerThread], xb[kPerThread];
  int g = blockIdx.x;
  if (g >= total) return;
  rowstats_load<VEC4>(p, g, xa);
  for (;;) {
    const int g1 = g + (int)gridDim.x;
    if (g1 < total) rowstats_load<VEC4>(p, g1, xb);
    rowstats_chunk<MODE, VEC4>(p, g, xa, sm, si, sd);
    if (g1 >= total) break;
    const int g2 = g1 + (int)gridDim.x;
    if (g2 < total) rowstats_load<VEC4>(p, g2, xa);
    rowstats_chunk<MODE, VEC4>(p, g1, xb, sm, si, sd);
    if (g2 >= total) break;
    g = g2;
  }
}

// log-normaliser of row `prow` from its chunk statistics, by one wave (lane k
// takes chunks k, k+64, ...); every lane gets it.
__device__ __forceinline__ double row_lse64(const AccParams& p, int prow) {
  const int lane = threadIdx.x & 63;
  const RowPart* pr = p.part + (size_t)prow * p.nchunk;
  float M = -INFINITY;
  for (int k = lane; k < p.nchunk; k += 64) M = fmaxf(M, pr[k].m);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  double Z = 0.0;
  for (int k = lane; k < p.nchunk; k += 64) {
    const RowPart q = pr[k];
    if (q.m != -INFINITY) Z += exp((double)q.m - (double)M) * q.s;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) Z += __shfl_xor(Z, off);
  return (double)M + log(Z);
}

// ---------------------------------------------------------------------------
// Relaxed acceptance: chunk sums of the Jensen-Shannon divergence terms of one
// drafted row pair (grid = drafted rows x vocab chunks), the JS distance
// between the draft and target distributions being what decides whether a
// draft token is close enough (the LLM inference handbook, section "AdaSD").
// With l = ln((p_j + q_j)/2) the divergence is half the sum over j of
// t_j = p_j (ln p_j - l) + q_j (ln q_j - l).  With x = |ln p_j - ln q_j|,
// u = x/2 and P the larger of p_j, q_j, t_j = 2 sqrt(p_j q_j) (u sinh u -
// cosh u ln cosh u), whose series is sqrt(p_j q_j) (u^2 + u^6/72 - u^8/360 +
// 443 u^10/604800 - 559 u^12/2721600 + ...) (relative error below 2e-8 for
// x < 1); for x >= 1, t_j = P ((1 + e^-x) h - x e^-x) with h = ln 2 -
// ln(1 + e^-x), which has no cancellation there and gives P ln 2 when one side
// is zero.  Both forms come from P and z = e^(-x/2) (sqrt(p_j q_j) = P z,
// e^-x = z^2), so an element costs three transcendentals and no divergent
// branch.  Terms in fp32 with the hardware exp2/log2, sums in fp64.
template <int VEC4>
__global__ __launch_bounds__(kAccThreads) void accept_jsd(AccParams p) {
  __shared__ double sd[4];
  __shared__ double s_lse[2];
  const int r = blockIdx.x / p.nchunk;          // drafted row
  const int c = blockIdx.x - r * p.nchunk;
  const int tid = threadIdx.x;
  // its sequence: the last b with q_start[b] - b <= r
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.q_start[mid] - mid <= r) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int t0 = p.q_start[b], D = seq_d(p, b), d0 = t0 - b;
  const int i = r - d0;
  if (!seq_ok(p, t0, D, d0) || i < 0 || i >= D) {
    if (tid == 0) p.jsp[(size_t)r * p.nchunk + c] = 0.0;
    return;
  }
  if (tid < 64) {
    const double lp = row_lse64(p, t0 + i);
    const double lq = row_lse64(p, p.T + r);
    if (tid == 0) { s_lse[0] = lp; s_lse[1] = lq; }
  }
  __syncthreads();
  const float lse_p = (float)s_lse[0], lse_q = (float)s_lse[1];
  const float dlse = (float)(s_lse[0] - s_lse[1]);
  const int j0 = c * kChunk;
  float tl[kPerThread], dl[kPerThread];
  load_chunk<VEC4>(p.target + (size_t)(t0 + i) * p.V, j0, p.V, tl);
  load_chunk<VEC4>(p.draft + (size_t)r * p.V, j0, p.V, dl);
  double acc = 0.0;
#pragma unroll
  for (int k0 = 0; k0 < kPerThread; k0 += 8) {
    float part = 0.f;                            // eight terms in fp32, then into the fp64 sum
#pragma unroll
    for (int k = k0; k < k0 + 8; ++k) {
      const float a = tl[k] - lse_p, bq = dl[k] - lse_q;     // ln p_j, ln q_j
      const float hi = fmaxf(a, bq);
      const float x = fabsf((tl[k] - dl[k]) - dlse);          // |ln p_j - ln q_j| (inf: one side 0)
      const float P = fast_exp2(hi * kLog2e);
      const float z = fast_exp2(x * (-0.5f * kLog2e));
      const float u = 0.5f * x, u2 = u * u;
      const float poly = u2 * (1.f + u2 * u2 * (1.f / 72.f + u2 * (-1.f / 360.f + u2 * (443.f / 604800.f +
                                                                     u2 * (-559.f / 2721600.f)))));
      const float y = z * z;
      const float h = 0.69314718f * (1.f - __log2f(1.f + y));
      const float tb = (1.f + y) * h - (y > 0.f ? y * x : 0.f);
      const float t = P * (x < 1.f ? z * poly : tb);
      if (hi != -INFINITY) part += t;                         // (p_j = q_j = 0: no term)
    }
    acc += (double)part;
  }
  acc = block_sum(acc, sd);
  if (tid == 0) p.jsp[(size_t)r * p.nchunk + c] = acc;
}

// Entropy (nats) and JS distance of drafted row r, from the chunk sums, by the
// 16 lanes of a group (lane k takes chunks k, k+16, ...; every lane of the
// group must call it, and each gets the result): H = log S0 - S1/S0 with
// S0 = sum_c exp(m_c - M) s_c and S1 = sum_c exp(m_c - M) (e_c + (m_c - M) s_c);
// JS = sqrt(JSD) with JSD half the sum of the chunk sums of the divergence
// terms.
__device__ __forceinline__ void row_relaxed_stats16(const AccParams& p, int r, int lane16, double& H, double& js) {
  const RowPart* pr = p.part + (size_t)(p.T + r) * p.nchunk;
  const double* e = p.ent + (size_t)r * p.nchunk;
  const double* jp = p.jsp + (size_t)r * p.nchunk;
  float M = -INFINITY;
  for (int k = lane16; k < p.nchunk; k += 16) M = fmaxf(M, pr[k].m);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  double S0 = 0.0, S1 = 0.0, J = 0.0;
  for (int k = lane16; k < p.nchunk; k += 16) {
    const RowPart q = pr[k];
    if (q.m != -INFINITY) {
      const double w = exp((double)q.m - (double)M);
      S0 += w * q.s;
      S1 += w * (e[k] + ((double)q.m - (double)M) * q.s);
    }
    J += jp[k];
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    S0 += __shfl_xor(S0, off);
    S1 += __shfl_xor(S1, off);
    J += __shfl_xor(J, off);
  }
  H = log(S0) - S1 / S0;
  js = sqrt(fmax(0.0, 0.5 * J));
}

// ---------------------------------------------------------------------------
// The greedy decision of sequence b (one workgroup); amax: LDS for its D+1 row
// argmaxes.  LOSSY: a draft also passes when the JS distance of its rows is at
// most tau, and the rows' entropy and JS distance are written out.
template <bool LOSSY>
__device__ __forceinline__ void decide_seq(const AccParams& p, int b, int* amax) {
  __shared__ RowPart stage[kDecideSlots];
  __shared__ int first_fail;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, D, d0)) {
    if (tid == 0) p.accept_len[b] = 0;
    return;
  }

  const int nrows = D + 1;                      // target rows t0 .. t0+D
  const int rows_per_pass = max(1, kDecideSlots / p.nchunk);
  for (int r0 = 0; r0 < nrows; r0 += rows_per_pass) {
    const int nr = min(rows_per_pass, nrows - r0);
    __syncthreads();
    for (int e = tid; e < nr * p.nchunk; e += kAccThreads)
      stage[e] = p.part[(size_t)(t0 + r0 + e / p.nchunk) * p.nchunk + (e % p.nchunk)];
    __syncthreads();
    for (int rr = tid; rr < nr; rr += kAccThreads) {
      const RowPart* pr = stage + rr * p.nchunk;
      float M = -INFINITY;
      int ai = INT_MAX;
      for (int c = 0; c < p.nchunk; ++c)
        if (better(pr[c].m, pr[c].idx, M, ai)) { M = pr[c].m; ai = pr[c].idx; }
      amax[r0 + rr] = ai;
    }
  }
  if (tid == 0) first_fail = D;
  __syncthreads();

  if constexpr (LOSSY) {
    // relaxed: a group of 16 lanes per draft, which also passes when the JS
    // distance of its rows is at most tau
    const int lane16 = tid & 15, grp = tid >> 4;
    for (int i0 = 0; i0 < D; i0 += kAccThreads / 16) {
      const int i = i0 + grp;
      if (i < D) {   // (uniform over the group's 16 lanes)
        double H, js;
        row_relaxed_stats16(p, d0 + i, lane16, H, js);
        if (lane16 == 0) {
          const int x = p.tokens[d0 + i];
          if (p.out_ent) p.out_ent[d0 + i] = (float)H;
          if (p.out_js) p.out_js[d0 + i] = (float)js;
          const bool pass = x >= 0 && x < p.V && (x == amax[i] || js <= (double)p.tau);
          if (!pass) atomicMin(&first_fail, i);
        }
      }
    }
  } else {
    for (int i = tid; i < D; i += kAccThreads) {
      const int x = p.tokens[d0 + i];
      const bool pass = x >= 0 && x < p.V && x == amax[i];
      if (!pass) atomicMin(&first_fail, i);
    }
  }
  __syncthreads();
  const int n = first_fail;
  for (int k = tid; k <= D; k += kAccThreads) p.out_tokens[t0 + k] = k < n ? p.tokens[d0 + k] : k == n ? amax[n] : -1;
  if (tid == 0) p.accept_len[b] = n + 1;
}

template <bool LOSSY>
__global__ __launch_bounds__(kAccThreads) void accept_decide(AccParams p) {
  extern __shared__ int amax[];                 // [D+1] row argmaxes
  decide_seq<LOSSY>(p, blockIdx.x, amax);
}

// ---------------------------------------------------------------------------
// Greedy acceptance of a draft tree (one workgroup per sequence).  Node i of
// sequence b (i = 0..T, node 0 the root) is verify row t0+i; nodes 1..T carry
// tokens[d0+i-1] and parents[d0+i-1] < i.  Node c is accepted iff its parent p
// is, and its token equals the top token of row p; the deepest accepted node
// (the lowest index among equal depths) ends the path, which is emitted with
// the target's top token at that node after it (the LLM inference handbook,
// section "Medusa": the longest accepted candidate prefix moves on).
__global__ __launch_bounds__(kAccThreads) void accept_tree(AccParams p, const int* parents, int* out_nodes) {
  extern __shared__ int amax[];                  // [T+1]: each node's top token
  __shared__ RowPart stage[kDecideSlots];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int T = seq_d(p, b);
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, T, d0)) {
    if (tid == 0) p.accept_len[b] = 0;
    return;
  }

  const int nrows = T + 1;
  const int rows_per_pass = max(1, kDecideSlots / p.nchunk);
  for (int r0 = 0; r0 < nrows; r0 += rows_per_pass) {
    const int nr = min(rows_per_pass, nrows - r0);
    __syncthreads();
    for (int e = tid; e < nr * p.nchunk; e += kAccThreads)
      stage[e] = p.part[(size_t)(t0 + r0 + e / p.nchunk) * p.nchunk + (e % p.nchunk)];
    __syncthreads();
    for (int rr = tid; rr < nr; rr += kAccThreads) {
      const RowPart* pr = stage + rr * p.nchunk;
      float M = -INFINITY;
      int ai = INT_MAX;
      for (int c = 0; c < p.nchunk; ++c)
        if (better(pr[c].m, pr[c].idx, M, ai)) { M = pr[c].m; ai = pr[c].idx; }
      amax[r0 + rr] = ai;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  // One wave decides: lane i holds node i.  A node matches when its token is the
  // top token of its parent's row; it is accepted when every node on its root
  // path matches, i.e. when its ancestor mask (built by pointer jumping, as for
  // tree attention) has no non-matching node.  A parent out of [0, i) is the root.
  const int lane = tid;
  int up = 0, x = -1;
  bool match = lane == 0;
  if (lane >= 1 && lane <= T) {
    const int q = parents[d0 + lane - 1];
    up = (q >= 0 && q < lane) ? q : 0;
    x = p.tokens[d0 + lane - 1];
    match = x >= 0 && x < p.V && x == amax[up];
  }
  const unsigned long long ok = __ballot(match);
  unsigned long long m = 1ull << lane;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const unsigned long long mu = __shfl(m, up);
    const int uu = __shfl(up, up);
    m |= mu;
    up = uu;
  }
  const int depth = __popcll(m) - 1;
  // the deepest accepted node, the lowest index among equal depths
  int key = (lane <= T && (m & ~ok) == 0) ? depth * 64 + (63 - lane) : -1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off));
  const int best = 63 - (key & 63);
  const int L = key >> 6;
  const unsigned long long path = __shfl(m, best);
  if (lane >= 1 && ((path >> lane) & 1ull)) {     // (node indices grow along a path)
    p.out_tokens[t0 + depth - 1] = x;
    out_nodes[t0 + depth - 1] = lane;
  }
  if (lane == 0) {
    p.out_tokens[t0 + L] = amax[best];
    p.accept_len[b] = L + 1;
  }
  for (int k = lane; k <= T; k += 64) {
    if (k > L) p.out_tokens[t0 + k] = -1;
    if (k >= L) out_nodes[t0 + k] = -1;
  }
}

// fp64 weights of one token of the sampling row from its target logit tl and
// draft logit dl: pj = p(j); w = max(0, p(j) - q(j)) at a rejection, p(j) when
// every draft passed.  A token past the vocabulary comes in as -inf (weight 0).
__device__ __forceinline__ void sample_weight(float tl, float dl, const SeqState& st, double& w, double& pj) {
  pj = exp((double)tl - st.lse_p);
  w = st.residual ? fmax(0.0, pj - exp((double)dl - st.lse_q)) : pj;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

// log-normaliser log(sum_x exp(l_x)) of row `prow` from its chunk statistics,
// merged by the 16 lanes of a group (lane k takes chunks k, k+16, ...): the row
// max M over the chunk maxima, then log(sum_c exp(m_c - M) s_c) + M in fp64.
// Every lane of the group must call it; each gets the result.
__device__ __forceinline__ double row_lse16(const AccParams& p, int prow, int lane16) {
  const RowPart* pr = p.part + (size_t)prow * p.nchunk;
  RowPart a0, a1;
  a0.m = a1.m = -INFINITY;
  a0.s = a1.s = 0.0;
  if (lane16 < p.nchunk) a0 = pr[lane16];
  if (lane16 + 16 < p.nchunk) a1 = pr[lane16 + 16];
  float M = fmaxf(a0.m, a1.m);
  for (int k = lane16 + 32; k < p.nchunk; k += 16) M = fmaxf(M, pr[k].m);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  double Z = 0.0;
  if (a0.m != -INFINITY) Z += exp((double)a0.m - (double)M) * a0.s;
  if (a1.m != -INFINITY) Z += exp((double)a1.m - (double)M) * a1.s;
  for (int k = lane16 + 32; k < p.nchunk; k += 16) {
    const RowPart q = pr[k];
    if (q.m != -INFINITY) Z += exp((double)q.m - (double)M) * q.s;
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) Z += __shfl_xor(Z, off);
  return (double)M + log(Z);
}

// ---------------------------------------------------------------------------
// The stochastic decision of sequence b and the sums of its chunks c0, c0 +
// cstep, ... (one workgroup; the workgroup with c0 = 0 writes the decision).
template <bool LOSSY>
__device__ __forceinline__ void finish_seq(const AccParams& p, int b, int c0, int cstep) {
  __shared__ double sd[4];
  __shared__ int s_fail, s_have;
  __shared__ double s_lp, s_lq;
  const int c = c0;
  const int tid = threadIdx.x;
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, D, d0)) {
    if (c == 0 && tid == 0) p.accept_len[b] = 0;
    return;
  }

  // (0) the decision.  Group g (16 lanes) takes draft position i = r0 + g of
  // each pass: the log-normalisers of target row i and draft row i, then (lane
  // 0) the test of draft i: it passes when u_i < p(x_i) / q(x_i), evaluated as
  // exp((l_p - LSE_p) - (l_q - LSE_q)) in fp64.  Row D has no draft row.
  const int lane16 = tid & 15, grp = tid >> 4;
  const float u_sample = c == 0 && tid == 0 ? p.uniforms[t0 + D] : 0.f;   // (for the draw; loaded early)
  if (tid == 0) { s_fail = D; s_have = 0; }
  __syncthreads();
  double my_lp = 0.0, my_lq = 0.0;
  int my_i = -1;
  for (int r0 = 0; r0 <= D; r0 += kAccThreads / 16) {
    const int i = r0 + grp;
    const bool live = i <= D;
    const bool test = i < D && lane16 == 0;
    int x = -1;
    float ut = 0.f;
    if (test) { x = p.tokens[d0 + i]; ut = p.uniforms[t0 + i]; }
    const bool inv = x >= 0 && x < p.V;
    float tl = 0.f, dl = 0.f;
    if (test && inv) { tl = p.target[(size_t)(t0 + i) * p.V + x]; dl = p.draft[(size_t)(d0 + i) * p.V + x]; }
    const double lp = row_lse16(p, t0 + (live ? i : 0), lane16);
    // (draft rows d0 .. d0+D-1 exist only for D > 0, a condition uniform over the workgroup)
    const double lq = D > 0 ? row_lse16(p, p.T + d0 + min(i, D - 1), lane16) : 0.0;
    if (live) { my_lp = lp; my_lq = lq; my_i = i; }
    // relaxed: the drafted row's entropy and JS distance, by every lane of the group
    double H = 0.0, js = 0.0;
    if constexpr (LOSSY) {
      if (D > 0) row_relaxed_stats16(p, d0 + min(i, D - 1), lane16, H, js);
    }
    if (test) {
      const double r = exp(((double)tl - lp) - ((double)dl - lq));
      bool pass = inv && (double)ut < r;
      if constexpr (LOSSY) {
        // the draft also passes when the JS distance of its rows is at most tau
        if (c0 == 0) {
          if (p.out_ent) p.out_ent[d0 + i] = (float)H;
          if (p.out_js) p.out_js[d0 + i] = (float)js;
        }
        pass = inv && ((double)ut < r || js <= (double)p.tau);
      }
      if (!pass) atomicMin(&s_fail, i);
    }
  }
  __syncthreads();
  const int n = s_fail;
  if (my_i == n && lane16 == 0) { s_lp = my_lp; s_lq = my_lq; s_have = 1; }
  __syncthreads();
  if (!s_have && grp == 0) {           // n fell in an earlier pass: merge its rows again
    const double lp = row_lse16(p, t0 + n, lane16);
    const double lq = n < D ? row_lse16(p, p.T + d0 + n, lane16) : 0.0;
    if (lane16 == 0) { s_lp = lp; s_lq = lq; }
  }
  __syncthreads();
  if (c == 0) {
    for (int k = tid; k <= D; k += kAccThreads)
      if (k != n) p.out_tokens[t0 + k] = k < n ? p.tokens[d0 + k] : -1;   // k == n: the sample (accept_draw)
    if (tid == 0) {
      p.accept_len[b] = n + 1;
      p.seqrec[b] = SeqRec{s_lp, n < D ? s_lq : 0.0, n, u_sample};
    }
  }
  SeqState st;
  st.n = n;
  st.residual = n < D;
  st.lse_p = s_lp;
  st.lse_q = n < D ? s_lq : 0.0;

  // (1) fp64 sums of the workgroup's chunks (c = blockIdx.x, + gridDim.x, ...).
  // Thread t takes the 16 consecutive logits j0 .. j0+15 of a chunk (all
  // loaded before any arithmetic): the weight of token j is max(0, p_j - q_j)
  // at a rejection, p_j when every draft passed.  The thread publishes its own
  // sums (residual, p) and the workgroup the chunk's, for accept_draw.
  const float* prow = p.target + (size_t)(t0 + n) * p.V;
  const float* qrow = p.draft + (size_t)(d0 + (n < D ? n : 0)) * p.V;
  for (int c = c0; c < p.nschunk; c += cstep) {
    const int j0 = c * kSChunk + tid * kSPerThread;
    float tl[kSPerThread], dl[kSPerThread];
    if (p.vec4 && j0 + kSPerThread <= p.V) {
#pragma unroll
      for (int k = 0; k < kSPerThread / 4; ++k) {
        const f32x4 v = *(const f32x4*)(prow + j0 + 4 * k);
        const f32x4 u = st.residual ? *(const f32x4*)(qrow + j0 + 4 * k) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) { tl[4 * k + e] = v[e]; dl[4 * k + e] = u[e]; }
      }
    } else {
#pragma unroll
      for (int e = 0; e < kSPerThread; ++e) {
        const bool in = j0 + e < p.V;
        tl[e] = in ? prow[j0 + e] : -INFINITY;
        dl[e] = in && st.residual ? qrow[j0 + e] : -INFINITY;
      }
    }
    double tw = 0.0, tp = 0.0;
#pragma unroll
    for (int e = 0; e < kSPerThread; ++e) {
      double w, pj;
      sample_weight(tl[e], dl[e], st, w, pj);
      tw += w;
      tp += pj;
    }
    double* dst = p.rsub + (((size_t)b * p.nschunk + c) * kAccThreads + tid) * 2;
    *(f64x2*)dst = f64x2{tw, tp};
    const double zw = block_sum(tw, sd);
    const double zp = block_sum(tp, sd);
    if (tid == 0) {
      double* cs = p.rsum + ((size_t)b * p.nschunk + c) * 2;
      *(f64x2*)cs = f64x2{zw, zp};
    }
  }
}

template <bool LOSSY>
__global__ __launch_bounds__(kAccThreads) void accept_finish(AccParams p) {
  finish_seq<LOSSY>(p, blockIdx.y, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// (2) one workgroup per stochastic sequence draws the token from the sums
// accept_finish left: the first token whose inclusive prefix sum of weights
// exceeds T = u * Z, found in three levels (chunk, 16-token slice, token).
// Where rounding leaves T past every prefix of a level, the level takes its
// last element with weight > 0.
__device__ __forceinline__ void draw_seq(const AccParams& p, int b) {
  __shared__ double s_wtot[4];
  __shared__ int s_chunk, s_usep, s_slice, s_slice_last;
  __shared__ double s_base, s_slice_base, s_T;
  __shared__ float s_tl[kSPerThread], s_dl[kSPerThread];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // Two memory round trips.  The first: the sequence's rows, its decision and
  // (wave 0) the chunk sums.
  const double* rs = p.rsum + (size_t)b * p.nschunk * 2;
  f64x2 r0 = {0.0, 0.0};
  if (wave == 0 && lane < p.nschunk) r0 = *(const f64x2*)(rs + 2 * lane);
  const SeqRec rec = p.seqrec[b];
  const int t0 = p.q_start[b];
  const int D = seq_d(p, b);
  const int d0 = t0 - b;
  if (!seq_ok(p, t0, D, d0)) return;   // (accept_finish wrote AL = 0)
  const int n = min(max(rec.n, 0), D);
  SeqState st;
  st.n = n;
  st.residual = n < D;
  st.lse_p = rec.lse_p;
  st.lse_q = rec.lse_q;
  const float* prow = p.target + (size_t)(t0 + n) * p.V;
  const float* qrow = p.draft + (size_t)(d0 + (n < D ? n : 0)) * p.V;
  if (wave == 0) {
    // level 1 (one wave): totals, T, and the chunk
    const double vw0 = r0[0], vp0 = r0[1];
    double sw = vw0, sp = vp0;
    for (int k = lane + 64; k < p.nschunk; k += 64) { sw += rs[2 * k]; sp += rs[2 * k + 1]; }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) { sw += __shfl_xor(sw, off); sp += __shfl_xor(sp, off); }
    const int usep = !(sw > 0.0);                 // the residual has no mass: sample p
    const double T = (double)rec.u * (usep ? sp : sw);
    double carry = 0.0, base = -INFINITY;
    int chunk = -1, lastpos = -1;
    for (int kb = 0; kb < p.nschunk; kb += 64) {
      const int k = kb + lane;
      const double v = kb == 0 ? (usep ? vp0 : vw0) : (k < p.nschunk ? rs[2 * k + usep] : 0.0);
      const double incl = wave_incl_scan(v);
      double excl = __shfl_up(incl, 1);
      if (lane == 0) excl = 0.0;
      const unsigned long long hit = __ballot(k < p.nschunk && carry + incl > T);
      const unsigned long long pos = __ballot(v > 0.0);
      if (pos) lastpos = kb + 63 - __clzll(pos);
      if (hit) {
        const int l = __ffsll(hit) - 1;
        chunk = kb + l;
        base = carry + __shfl(excl, l);
        break;
      }
      carry += __shfl(incl, 63);
    }
    if (chunk < 0) chunk = max(lastpos, 0);       // base stays -inf: every later level falls back
    if (lane == 0) { s_chunk = chunk; s_base = base; s_T = T; s_usep = usep; s_slice = INT_MAX; s_slice_last = -1; }
  }
  __syncthreads();
  const int chunk = s_chunk;
  const double T = s_T;
  const int usep = s_usep;
  // The second: each thread's sums in the chosen chunk, and its 16 logits there
  // (level 3 needs only the chosen slice's, but they are then already here).
  const f64x2 rv = *(const f64x2*)(p.rsub + (((size_t)b * p.nschunk + chunk) * kAccThreads + tid) * 2);
  const int j0 = chunk * kSChunk + tid * kSPerThread;
  float tl[kSPerThread], dl[kSPerThread];
  if (p.vec4 && j0 + kSPerThread <= p.V) {
#pragma unroll
    for (int k = 0; k < kSPerThread / 4; ++k) {
      const f32x4 a = *(const f32x4*)(prow + j0 + 4 * k);
      const f32x4 q = st.residual ? *(const f32x4*)(qrow + j0 + 4 * k) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) { tl[4 * k + e] = a[e]; dl[4 * k + e] = q[e]; }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSPerThread; ++e) {
      const bool in = j0 + e < p.V;
      tl[e] = in ? prow[j0 + e] : -INFINITY;
      dl[e] = in && st.residual ? qrow[j0 + e] : -INFINITY;
    }
  }
  // level 2 (four waves): the 16-token slice inside the chunk, from the thread sums
  {
    const double v = usep ? rv[1] : rv[0];
    const double incl = wave_incl_scan(v);
    if (lane == 63) s_wtot[wave] = incl;
    __syncthreads();
    double carry = s_base;
    for (int w = 0; w < wave; ++w) carry += s_wtot[w];
    if (carry + incl > T) atomicMin(&s_slice, tid);
    if (v > 0.0) atomicMax(&s_slice_last, tid);
    __syncthreads();
    if (tid == s_slice) s_slice_base = carry + (incl - v);
    if (tid == (s_slice != INT_MAX ? s_slice : max(s_slice_last, 0))) {
#pragma unroll
      for (int e = 0; e < kSPerThread; ++e) { s_tl[e] = tl[e]; s_dl[e] = dl[e]; }
    }
  }
  __syncthreads();
  if (wave == 0) {
    // level 3 (one wave): the token inside the slice, by a sequential prefix sum
    const int slice = s_slice != INT_MAX ? s_slice : max(s_slice_last, 0);
    const double base = s_slice != INT_MAX ? s_slice_base : -INFINITY;
    if (usep) st.residual = 0;
    const int js = chunk * kSChunk + slice * kSPerThread;
    double w = 0.0;
    if (lane < kSPerThread) {   // (past the vocabulary the logits are -inf: weight 0)
      double pj;
      sample_weight(s_tl[lane], st.residual ? s_dl[lane] : -INFINITY, st, w, pj);
    }
    double C = base;
    int tok = -1, last = -1;
#pragma unroll
    for (int e = 0; e < kSPerThread; ++e) {
      const double we = __shfl(w, e);
      C += we;
      if (tok < 0 && C > T) tok = js + e;
      if (we > 0.0) last = js + e;
    }
    if (tok < 0) tok = last >= 0 ? last : js;
    if (lane == 0) p.out_tokens[t0 + n] = tok;
  }
}

__global__ __launch_bounds__(kAccThreads) void accept_draw(AccParams p) { draw_seq(p, blockIdx.x); }

// The stochastic decision and the draw of sequence b in one workgroup, for
// calls where accept_finish would run a single workgroup per sequence anyway
// (one sampling chunk, or enough sequences): a workgroup barrier where the
// two-kernel path has a launch boundary, the same code on the same data.
template <bool LOSSY>
__global__ __launch_bounds__(kAccThreads) void accept_finish_draw(AccParams p) {
  finish_seq<LOSSY>(p, blockIdx.x, 0, 1);
  __syncthreads();
  draw_seq(p, blockIdx.x);
}

// Small vocabularies (V <= kSmallV, so one chunk per row and a whole row in
// kSmallPL logits per lane): one workgroup per sequence does the whole call.
// Each wave makes the statistics of whole rows on its own (wave shuffles, no
// workgroup barrier), the four waves taking the sequence's rows in turn, so
// the rows run in parallel; then the decision and (stochastic) the draw run as
// in accept_finish_draw.  The fp64 row sums add the same fp32 terms in another
// order than accept_rowstats.
constexpr int kSmallV = 2048;
constexpr int kSmallPL = kSmallV / 64;

template <int VEC4>
__device__ __forceinline__ void small_row_load(const float* src, int V, float (&x)[kSmallPL]) {
  const int lane = threadIdx.x & 63;
  if (VEC4) {   // lane's logits (i*64 + lane)*4 + e; V % 4 == 0, so a vector lies wholly inside or past the row
#pragma unroll
    for (int i = 0; i < kSmallPL / 4; ++i) {
      const int j = (i * 64 + lane) * 4;
      const f32x4 v = j < V ? __builtin_nontemporal_load((const f32x4*)(src + j))
                            : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i * 4 + e] = v[e];
    }
  } else {      // lane's logits i*64 + lane
#pragma unroll
    for (int i = 0; i < kSmallPL; ++i) {
      const int j = i * 64 + lane;
      x[i] = j < V ? src[j] : -INFINITY;
    }
  }
}

// The row's statistics by one wave (every lane returns them): greedy, the
// lowest-index maximum; stochastic, the maximum and the fp64 sum of exp(x - m).
template <bool STOCH, int VEC4>
__device__ __forceinline__ RowPart small_row_stats(const float (&x)[kSmallPL], int V) {
  const int lane = threadIdx.x & 63;
  RowPart r;
  r.idx = 0;
  r.s = 0.0;
  float m = -INFINITY;
  if constexpr (!STOCH) {
    int idx = INT_MAX;   // (increasing indices in k; a row of -inf reports its first index)
#pragma unroll
    for (int k = 0; k < kSmallPL; ++k) {
      const int j = VEC4 ? ((k >> 2) * 64 + lane) * 4 + (k & 3) : k * 64 + lane;
      if (x[k] > m || (idx == INT_MAX && j < V)) { m = x[k]; idx = j; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float om = __shfl_xor(m, off);
      const int oi = __shfl_xor(idx, off);
      if (better(om, oi, m, idx)) { m = om; idx = oi; }
    }
    r.idx = idx;
  } else {
#pragma unroll
    for (int k = 0; k < kSmallPL; ++k) m = fmaxf(m, x[k]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    double sum = 0.0;
    if (m != -INFINITY) {
      const float ml = m * kLog2e;
#pragma unroll
      for (int k0 = 0; k0 < kSmallPL; k0 += 8) {
        float a = 0.f;
#pragma unroll
        for (int k = k0; k < k0 + 8; ++k) a += fast_exp2(fmaf(x[k], kLog2e, -ml));
        sum += (double)a;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    }
    r.s = sum;
  }
  r.m = m;
  return r;
}

template <bool STOCH, int VEC4>
__global__ __launch_bounds__(kAccThreads) void accept_small(AccParams p) {
  extern __shared__ int amax[];                 // greedy: [max_draft + 1] row argmaxes
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int t0 = p.q_start[b], D = seq_d(p, b), d0 = t0 - b;
  if (seq_ok(p, t0, D, d0)) {                   // (otherwise the decision writes AL = 0)
    // target rows t0 .. t0+D, then (stochastic) draft rows d0 .. d0+D-1
    const int nrows = STOCH ? 2 * D + 1 : D + 1;
    for (int k = wave; k < nrows; k += kAccThreads / 64) {
      const int row = k <= D ? t0 + k : p.T + d0 + (k - D - 1);
      const float* src = row < p.T ? p.target + (size_t)row * p.V : p.draft + (size_t)(row - p.T) * p.V;
      float x[kSmallPL];
      small_row_load<VEC4>(src, p.V, x);
      const RowPart r = small_row_stats<STOCH, VEC4>(x, p.V);
      if ((threadIdx.x & 63) == 0) p.part[row] = r;   // (one chunk per row)
    }
  }
  __syncthreads();
  if constexpr (STOCH) {
    finish_seq<false>(p, b, 0, 1);
    __syncthreads();
    draw_seq(p, b);
  } else {
    decide_seq<false>(p, b, amax);
  }
}

struct AccLayout {
  size_t part_off, seqrec_off, rsum_off, rsub_off, ent_off, jsp_off, total;
  int nchunk, nschunk;
};

// Row statistics cover the target rows, and the draft rows too when the
// acceptance is stochastic or relaxed; the relaxed rule adds two chunk-sum
// arrays over the draft rows.
static AccLayout acc_layout(int B, int T, int V, int stochastic, int lossy) {
  AccLayout L;
  L.nchunk = (V + kChunk - 1) / kChunk;
  L.nschunk = (V + kSChunk - 1) / kSChunk;
  const size_t drows = (size_t)(T - B);
  const size_t rows = (stochastic || lossy) ? (size_t)T + drows : (size_t)T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.part_off = take(rows * L.nchunk * sizeof(RowPart));
  L.seqrec_off = take(stochastic ? (size_t)B * sizeof(SeqRec) : 0);
  L.rsum_off = take((size_t)B * L.nschunk * 2 * sizeof(double));
  L.rsub_off = take(stochastic ? (size_t)B * L.nschunk * kAccThreads * 2 * sizeof(double) : 0);
  L.ent_off = take(lossy ? drows * L.nchunk * sizeof(double) : 0);
  L.jsp_off = take(lossy ? drows * L.nchunk * sizeof(double) : 0);
  L.total = off;
  return L;
}

}  // namespace sdv

using namespace sdv;

size_t sdv_accept_workspace_bytes(int B, int T, int V, int stochastic, int lossy) {
  return acc_layout(B, T, V, stochastic, lossy).total;
}

hipError_t sdv_accept_launch(const SdAccLaunch& a) {
  const AccLayout L = acc_layout(a.B, a.T, a.V, a.stochastic, a.lossy);
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
  p.seqrec = (SeqRec*)(ws + L.seqrec_off);
  p.rsum = (double*)(ws + L.rsum_off);
  p.rsub = (double*)(ws + L.rsub_off);
  p.ent = a.lossy ? (double*)(ws + L.ent_off) : nullptr;
  p.jsp = a.lossy ? (double*)(ws + L.jsp_off) : nullptr;
  p.out_ent = a.lossy ? a.out_entropy : nullptr;
  p.out_js = a.lossy ? a.out_js : nullptr;
  p.tau = a.lossy ? a.js_threshold : -1.f;
  p.B = a.B;
  p.T = a.T;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.nschunk = L.nschunk;
  p.max_draft = a.max_draft;

  const bool need_draft = a.stochastic || a.lossy;
  const bool vec4 = (a.V % 4 == 0) && ((uintptr_t)a.target % 16 == 0) &&
                    (!need_draft || (uintptr_t)a.draft % 16 == 0);
  p.vec4 = vec4;
  if (!a.lossy && a.V <= kSmallV) {   // small vocabularies: the whole call in one launch
    if (a.stochastic) {
      if (vec4) accept_small<true, 1><<<a.B, kAccThreads, 0, a.stream>>>(p);
      else accept_small<true, 0><<<a.B, kAccThreads, 0, a.stream>>>(p);
    } else {
      const size_t lds = (size_t)(a.max_draft + 1) * sizeof(int);
      if (vec4) accept_small<false, 1><<<a.B, kAccThreads, lds, a.stream>>>(p);
      else accept_small<false, 0><<<a.B, kAccThreads, lds, a.stream>>>(p);
    }
    return hipGetLastError();
  }
  const size_t drows = (size_t)(a.T - a.B);
  const size_t rows = need_draft ? (size_t)a.T + drows : (size_t)a.T;
  const unsigned grid1 = (unsigned)(rows * L.nchunk);
  const unsigned rs_grid = std::max(1u, std::min(grid1, (unsigned)kRowstatsWGs));
  if (a.lossy && a.stochastic) {
    if (vec4) accept_rowstats<3, 1><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
    else accept_rowstats<3, 0><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
  } else if (a.lossy) {
    if (vec4) accept_rowstats<2, 1><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
    else accept_rowstats<2, 0><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
  }
  if (a.lossy) {
    if (drows > 0) {
      const unsigned grid2 = (unsigned)(drows * L.nchunk);
      if (vec4) accept_jsd<1><<<grid2, kAccThreads, 0, a.stream>>>(p);
      else accept_jsd<0><<<grid2, kAccThreads, 0, a.stream>>>(p);
    }
  } else if (a.stochastic) {
    if (vec4) accept_rowstats<1, 1><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
    else accept_rowstats<1, 0><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
  } else {
    if (vec4) accept_rowstats<0, 1><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
    else accept_rowstats<0, 0><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
  }
  if (a.stochastic) {
    // workgroups per sequence: all chunks, or about kFinishWGs / B in all when
    // that is fewer (each then takes several chunks)
    const int per_seq = std::max(1, std::min(L.nschunk, (kFinishWGs + a.B - 1) / std::max(a.B, 1)));
    if (per_seq == 1) {
      if (a.lossy) accept_finish_draw<true><<<a.B, kAccThreads, 0, a.stream>>>(p);
      else accept_finish_draw<false><<<a.B, kAccThreads, 0, a.stream>>>(p);
    } else {
      if (a.lossy) accept_finish<true><<<dim3(per_seq, a.B), kAccThreads, 0, a.stream>>>(p);
      else accept_finish<false><<<dim3(per_seq, a.B), kAccThreads, 0, a.stream>>>(p);
      accept_draw<<<a.B, kAccThreads, 0, a.stream>>>(p);
    }
  } else {
    const size_t lds = (size_t)(a.max_draft + 1) * sizeof(int);
    if (a.lossy) accept_decide<true><<<a.B, kAccThreads, lds, a.stream>>>(p);
    else accept_decide<false><<<a.B, kAccThreads, lds, a.stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t sdv_tree_accept_launch(const SdAccLaunch& a, const int32_t* parents, int32_t* out_nodes) {
  const AccLayout L = acc_layout(a.B, a.T, a.V, 0, 0);
  unsigned char* ws = (unsigned char*)a.workspace;
  AccParams p;
  p.target = a.target;
  p.draft = nullptr;
  p.tokens = a.tokens;
  p.q_start = a.q_start;
  p.uniforms = nullptr;
  p.accept_len = a.accept_len;
  p.out_tokens = a.out_tokens;
  p.part = (RowPart*)(ws + L.part_off);
  p.seqrec = nullptr;
  p.rsum = nullptr;
  p.rsub = nullptr;
  p.ent = p.jsp = nullptr;
  p.out_ent = p.out_js = nullptr;
  p.tau = -1.f;
  p.B = a.B;
  p.T = a.T;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.nschunk = L.nschunk;
  p.max_draft = a.max_draft;
  const bool vec4 = (a.V % 4 == 0) && ((uintptr_t)a.target % 16 == 0);
  p.vec4 = vec4;
  const unsigned grid1 = (unsigned)((size_t)a.T * L.nchunk);
  const unsigned rs_grid = std::max(1u, std::min(grid1, (unsigned)kRowstatsWGs));
  if (vec4) accept_rowstats<0, 1><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
  else accept_rowstats<0, 0><<<rs_grid, kAccThreads, 0, a.stream>>>(p, (int)grid1);
  accept_tree<<<a.B, kAccThreads, (size_t)(a.max_draft + 1) * sizeof(int), a.stream>>>(p, parents, out_nodes);
  return hipGetLastError();
}
