// A closed speculative-decoding loop on a bigram toy LM, on gfx950.
//
// Every round drafts D tokens per sequence, verifies them in one pass, keeps
// an accepted prefix, and measures the acceptance length; an exponential
// moving average (EMA) of it picks the next round's D among a few tiers, each
// tier with its own captured graph so that switching costs nothing (the LLM
// inference handbook, section on SGLang's adaptive speculative decoding).
// Only the speculation length changes, so the output is the target's own
// greedy decoding.
//
// One round (D fixed, verify rows laid out as B blocks of 1+D):
//   loop_draft   one wave per sequence: model-free n-gram drafter (the latest
//                earlier occurrence of the history's last k tokens, k = n .. 1,
//                proposes what followed it; -1 where history runs out)
//   loop_logits  the toy LM's forward pass: target row r = W[token of row r]
//   accept       the greedy accept/reject kernels of accept.hip
//   loop_append  one wave per sequence: append the AL emitted tokens
// The host reads the appended counts after each round (one stream
// synchronisation per round) and picks the next tier.

#include <math.h>

#include <algorithm>
#include <vector>

#include "common.h"

namespace sdv {

constexpr int kLoopSeqsPerBlock = 4;    // one wave per sequence

struct LoopParams {
  const float* W;        // [V, V] bigram logits
  int* hist;             // [B, max_len]
  int* len;              // [B]
  int* rows_in;          // [B (1+D)] token of each verify row
  int* draft;            // [B D]
  float* logits;         // [B (1+D), V]
  const int* accept_len; // [B]
  const int* out_tokens; // [B (1+D)]
  int* appended;         // [B]
  int B, V, max_len, ngram;
};

__global__ __launch_bounds__(64 * kLoopSeqsPerBlock) void loop_draft(LoopParams lp, int D) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kLoopSeqsPerBlock + (threadIdx.x >> 6);
  if (b >= lp.B) return;                       // (whole waves)
  const int* h = lp.hist + (size_t)b * lp.max_len;
  const int L = min(lp.len[b], lp.max_len);
  int* rows = lp.rows_in + (size_t)b * (1 + D);
  if (L < 1) {                                 // no history: nothing to verify from
    for (int i = lane; i <= D; i += 64) rows[i] = -1;
    for (int i = lane; i < D; i += 64) lp.draft[(size_t)b * D + i] = -1;
    return;
  }
  int found = -1, kf = 0;                       // start of the matched occurrence, its length
  if (D > 0) {
    for (int k = min(lp.ngram, L - 1); k >= 1 && found < 0; --k) {
      int suf[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) suf[t] = t < k ? h[L - k + t] : 0;
      // candidates j = L-k-1 down to 0, 64 at a time; the first chunk with a
      // match gives the largest j
      for (int top = L - k - 1; top >= 0 && found < 0; top -= 64) {
        const int j = top - lane;
        bool match = j >= 0;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (t < k && match) match = h[j + t] == suf[t];
        const unsigned long long m = __ballot(match);
        if (m) {
          found = top - (__ffsll(m) - 1);      // the lowest lane holds the largest j
          kf = k;
        }
      }
    }
  }
  if (lane == 0) rows[0] = h[L - 1];
  for (int i = lane; i < D; i += 64) {
    const int src = found + kf + i;
    const int tok = (found >= 0 && src < L) ? h[src] : -1;
    lp.draft[(size_t)b * D + i] = tok;
    rows[1 + i] = tok;
  }
}

// Target logits of every verify row: row r is W[rows_in[r]] (a token outside
// [0, V) reads row 0; its draft fails the test anyway).  grid = rows x ceil(V/1024).
__global__ __launch_bounds__(256) void loop_logits(LoopParams lp, int rows) {
  const int r = blockIdx.x / ((lp.V + 1023) / 1024);
  const int c = blockIdx.x - r * ((lp.V + 1023) / 1024);
  if (r >= rows) return;
  int tok = lp.rows_in[r];
  tok = (tok >= 0 && tok < lp.V) ? tok : 0;
  const float* src = lp.W + (size_t)tok * lp.V;
  float* dst = lp.logits + (size_t)r * lp.V;
  const int j = c * 1024 + threadIdx.x * 4;
  if ((lp.V & 3) == 0) {
    if (j < lp.V) *(f32x4*)(dst + j) = *(const f32x4*)(src + j);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e < lp.V) dst[j + e] = src[j + e];
  }
}

__global__ __launch_bounds__(64 * kLoopSeqsPerBlock) void loop_append(LoopParams lp, int D) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kLoopSeqsPerBlock + (threadIdx.x >> 6);
  if (b >= lp.B) return;
  const int L = lp.len[b];
  int a = lp.accept_len[b];
  if (L < 1 || a < 1 || a > 1 + D || L + a > lp.max_len) a = 0;   // full (or nothing to append)
  int* h = lp.hist + (size_t)b * lp.max_len;
  for (int i = lane; i < a; i += 64) h[L + i] = lp.out_tokens[(size_t)b * (1 + D) + i];
  if (lane == 0) {
    lp.len[b] = L + a;
    lp.appended[b] = a;
  }
}

__global__ void loop_qstart(int* q_start, int B, int D) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b <= B) q_start[b] = b * (1 + D);
}

struct LoopLayout {
  size_t qs_off, rows_off, draft_off, logits_off, al_off, out_off, app_off, acc_off, total;
};

static LoopLayout loop_layout(int B, int V, int ntiers, int dmax) {
  LoopLayout L;
  const size_t rmax = (size_t)B * (1 + dmax);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  L.qs_off = take((size_t)ntiers * (B + 1) * 4);
  L.rows_off = take(rmax * 4);
  L.draft_off = take((size_t)B * std::max(dmax, 1) * 4);
  L.logits_off = take(rmax * V * 4);
  L.al_off = take((size_t)B * 4);
  L.out_off = take(rmax * 4);
  L.app_off = take((size_t)B * 4);
  L.acc_off = take(sdv_accept_workspace_bytes(B, (int)rmax, V, 0, 0));
  L.total = off;
  return L;
}

}  // namespace sdv

using namespace sdv;

size_t sdv_loop_workspace_bytes(int B, int V, int ntiers, int dmax) {
  return loop_layout(B, V, ntiers, dmax).total;
}

namespace {

// one round at draft length D on `st`
hipError_t enqueue_round(const LoopParams& lp, unsigned char* ws, const LoopLayout& L, int tier, int D,
                         hipStream_t st) {
  const int B = lp.B;
  const int rows = B * (1 + D);
  const unsigned sb = (unsigned)((B + kLoopSeqsPerBlock - 1) / kLoopSeqsPerBlock);
  loop_draft<<<sb, 64 * kLoopSeqsPerBlock, 0, st>>>(lp, D);
  loop_logits<<<(unsigned)((size_t)rows * ((lp.V + 1023) / 1024)), 256, 0, st>>>(lp, rows);
  SdAccLaunch a{};
  a.target = lp.logits;
  a.draft = nullptr;
  a.tokens = lp.draft;
  a.q_start = (const int*)(ws + L.qs_off) + (size_t)tier * (B + 1);
  a.uniforms = nullptr;
  a.accept_len = (int*)(ws + L.al_off);
  a.out_tokens = (int*)(ws + L.out_off);
  a.workspace = ws + L.acc_off;
  a.B = B;
  a.T = rows;
  a.V = lp.V;
  a.max_draft = D;
  a.stochastic = 0;
  a.stream = st;
  hipError_t e = sdv_accept_launch(a);
  if (e != hipSuccess) return e;
  loop_append<<<sb, 64 * kLoopSeqsPerBlock, 0, st>>>(lp, D);
  return hipGetLastError();
}

}  // namespace

hipError_t sdv_closed_loop(const SdLoopLaunch& c) {
  const int dmax = *std::max_element(c.tiers, c.tiers + c.ntiers);
  const LoopLayout L = loop_layout(c.B, c.V, c.ntiers, dmax);
  unsigned char* ws = (unsigned char*)c.workspace;
  LoopParams lp;
  lp.W = c.W;
  lp.hist = c.hist;
  lp.len = c.len;
  lp.rows_in = (int*)(ws + L.rows_off);
  lp.draft = (int*)(ws + L.draft_off);
  lp.logits = (float*)(ws + L.logits_off);
  lp.accept_len = (const int*)(ws + L.al_off);
  lp.out_tokens = (const int*)(ws + L.out_off);
  lp.appended = (int*)(ws + L.app_off);
  lp.B = c.B;
  lp.V = c.V;
  lp.max_len = c.max_len;
  lp.ngram = c.ngram;
  for (int t = 0; t < c.ntiers; ++t)
    loop_qstart<<<(c.B + 256) / 256, 256, 0, c.stream>>>((int*)(ws + L.qs_off) + (size_t)t * (c.B + 1), c.B,
                                                         c.tiers[t]);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // one graph per tier, captured on a stream of our own and launched on the caller's
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  hipStream_t cs = nullptr;
  auto cleanup = [&]() {   // (teardown errors cannot change the call's result)
    for (auto x : execs) (void)hipGraphExecDestroy(x);
    for (auto g : graphs) (void)hipGraphDestroy(g);
    if (cs) (void)hipStreamDestroy(cs);
  };
  if (c.use_graphs) {
    e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    for (int t = 0; t < c.ntiers && e == hipSuccess; ++t) {
      hipGraph_t g = nullptr;
      e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
      if (e != hipSuccess) break;
      hipError_t eq = enqueue_round(lp, ws, L, t, c.tiers[t], cs);
      e = hipStreamEndCapture(cs, &g);
      if (e == hipSuccess) e = eq;
      if (g) graphs.push_back(g);
      if (e != hipSuccess) break;
      hipGraphExec_t x = nullptr;
      e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
      if (e == hipSuccess) execs.push_back(x);
    }
    if (e != hipSuccess) {
      cleanup();
      return e;
    }
  }

  // the rounds; after each, the appended counts come back and the EMA of the
  // mean AL picks the next tier (the smallest tier >= EMA, else the largest)
  double ema = 1.0;
  auto pick = [&](double v) {
    for (int t = 0; t < c.ntiers; ++t)
      if (c.tiers[t] >= v) return t;
    return c.ntiers - 1;
  };
  int tier = pick(ema);
  for (int s = 0; s < c.steps; ++s) {
    c.tier_trace[s] = c.tiers[tier];
    e = c.use_graphs ? hipGraphLaunch(execs[tier], c.stream) : enqueue_round(lp, ws, L, tier, c.tiers[tier], c.stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(c.al_trace + (size_t)s * c.B, lp.appended, (size_t)c.B * 4, hipMemcpyDeviceToHost, c.stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c.stream);
    if (e != hipSuccess) break;
    const int* al = c.al_trace + (size_t)s * c.B;
    long long sum = 0;
    int n = 0;
    for (int b = 0; b < c.B; ++b)
      if (al[b] > 0) { sum += al[b]; ++n; }
    if (n > 0) ema = (1.0 - c.ema_weight) * ema + c.ema_weight * ((double)sum / n);
    tier = pick(ema);
  }
  cleanup();
  return e;
}
