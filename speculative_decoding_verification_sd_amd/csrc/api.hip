// C ABI of the verify step: argument validation, workspace sizing and
// stream-ordered launches.  Nothing here allocates, frees or synchronises.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "sd_verify.h"
#include "common.h"

namespace {

thread_local std::string g_error;

sd_status fail(sd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

constexpr int kMaxRows = 256;   // G*(1+max_draft) handled by one workgroup

sd_status check_attn(const sd_attn_desc* d, int32_t total_q) {
  if (!d) return fail(SD_ERR_INVALID_ARG, "attention descriptor is NULL");
  if (d->num_seqs < 0) return fail(SD_ERR_INVALID_ARG, "num_seqs=%d must be >= 0", d->num_seqs);
  if (d->num_kv_heads < 1) return fail(SD_ERR_INVALID_ARG, "num_kv_heads=%d must be >= 1", d->num_kv_heads);
  if (d->group_size < 1) return fail(SD_ERR_INVALID_ARG, "group_size=%d must be >= 1", d->group_size);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SD_ERR_UNSUPPORTED, "head_dim=%d: supported values are 64 and 128", d->head_dim);
  if (d->page_size != 16) return fail(SD_ERR_UNSUPPORTED, "page_size=%d: only 16 is supported", d->page_size);
  if (d->max_pages_per_seq < 1) return fail(SD_ERR_INVALID_ARG, "max_pages_per_seq=%d must be >= 1", d->max_pages_per_seq);
  if ((long long)d->max_pages_per_seq * d->page_size > (1LL << 30))
    return fail(SD_ERR_UNSUPPORTED, "max_pages_per_seq*page_size exceeds 2^30 keys");
  if (d->num_pages < 1) return fail(SD_ERR_INVALID_ARG, "num_pages=%d must be >= 1", d->num_pages);
  if (d->max_draft < 0) return fail(SD_ERR_INVALID_ARG, "max_draft=%d must be >= 0", d->max_draft);
  if ((long long)d->group_size * (1LL + d->max_draft) > kMaxRows)
    return fail(SD_ERR_UNSUPPORTED, "group_size*(1+max_draft)=%lld exceeds %d rows per KV head",
                (long long)d->group_size * (1LL + d->max_draft), kMaxRows);
  if (!(d->softmax_scale >= 0.f) || !isfinite(d->softmax_scale))
    return fail(SD_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (d->out_dtype != SD_OUT_BF16 && d->out_dtype != SD_OUT_F32)
    return fail(SD_ERR_INVALID_ARG, "out_dtype=%d is not an sd_out_dtype", d->out_dtype);
  if (d->kv_chunk < 0 || d->kv_chunk % 64 != 0)
    return fail(SD_ERR_INVALID_ARG, "kv_chunk=%d must be 0 or a positive multiple of 64", d->kv_chunk);
  if (d->kv_chunk > 8192)
    return fail(SD_ERR_UNSUPPORTED, "kv_chunk=%d exceeds 8192 keys per work item", d->kv_chunk);
  if (d->v_layout != SD_V_KEY_MAJOR && d->v_layout != SD_V_DIM_MAJOR)
    return fail(SD_ERR_INVALID_ARG, "v_layout=%d is not an sd_v_layout", d->v_layout);
  if (total_q < d->num_seqs || (long long)total_q > (long long)d->num_seqs * (1LL + d->max_draft))
    return fail(SD_ERR_INVALID_ARG, "total_q=%d must lie in [num_seqs, num_seqs*(1+max_draft)] = [%d, %lld]",
                total_q, d->num_seqs, (long long)d->num_seqs * (1LL + d->max_draft));
  return SD_OK;
}

sd_status check_accept(const sd_accept_desc* d, int32_t total_q, bool lossy = false) {
  if (!d) return fail(SD_ERR_INVALID_ARG, "accept descriptor is NULL");
  if (d->num_seqs < 0) return fail(SD_ERR_INVALID_ARG, "num_seqs=%d must be >= 0", d->num_seqs);
  if (d->vocab < 1) return fail(SD_ERR_INVALID_ARG, "vocab=%d must be >= 1", d->vocab);
  if (d->max_draft < 0) return fail(SD_ERR_INVALID_ARG, "max_draft=%d must be >= 0", d->max_draft);
  if (d->max_draft > 4096) return fail(SD_ERR_UNSUPPORTED, "max_draft=%d exceeds 4096", d->max_draft);
  if (d->mode != SD_ACCEPT_GREEDY && d->mode != SD_ACCEPT_STOCHASTIC)
    return fail(SD_ERR_INVALID_ARG, "mode=%d is not an sd_accept_mode", d->mode);
  if (total_q < d->num_seqs || (long long)total_q > (long long)d->num_seqs * (1LL + d->max_draft))
    return fail(SD_ERR_INVALID_ARG, "total_q=%d must lie in [num_seqs, num_seqs*(1+max_draft)]", total_q);
  const long long rows = (d->mode == SD_ACCEPT_STOCHASTIC || lossy) ? 2LL * total_q - d->num_seqs : total_q;
  if (rows * ((d->vocab + 4095) / 4096) > 0x7fffffffLL)
    return fail(SD_ERR_UNSUPPORTED, "rows x vocab chunks exceeds the launch grid");
  return SD_OK;
}

size_t attn_ws(const sd_attn_desc* d) {
  return sdv_attn_workspace_bytes(d->num_seqs, d->num_kv_heads, d->group_size, d->head_dim,
                                  d->max_pages_per_seq, d->max_draft, d->kv_chunk);
}

size_t acc_ws(const sd_accept_desc* d, int32_t total_q, bool lossy = false) {
  return sdv_accept_workspace_bytes(d->num_seqs, total_q, d->vocab, d->mode == SD_ACCEPT_STOCHASTIC, lossy);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

sd_status run_attention(const sd_attn_desc* d, int32_t total_q, const void* q, const void* k,
                        const void* v, const int32_t* bt, const int32_t* kv_len, const int32_t* q_start,
                        void* out, void* ws, size_t ws_bytes, void* stream, const int32_t* parents = nullptr) {
  sd_status s = check_attn(d, total_q);
  if (s != SD_OK) return s;
  if (d->num_seqs == 0) return SD_OK;
  if (!q || !k || !v || !bt || !kv_len || !q_start || !out)
    return fail(SD_ERR_INVALID_ARG, "a required attention pointer is NULL");
  const size_t need = attn_ws(d);
  if (!ws || ws_bytes < need)
    return fail(SD_ERR_WORKSPACE, "attention workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws % 16 || (uintptr_t)q % 16 || (uintptr_t)k % 16 || (uintptr_t)v % 16 || (uintptr_t)out % 16)
    return fail(SD_ERR_INVALID_ARG, "q, caches, out and workspace must be 16-byte aligned");
  SdAttnLaunch a;
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.block_table = bt;
  a.kv_len = kv_len;
  a.q_start = q_start;
  a.parents = parents;
  a.out = out;
  a.workspace = ws;
  a.B = d->num_seqs;
  a.Hkv = d->num_kv_heads;
  a.G = d->group_size;
  a.head_dim = d->head_dim;
  a.max_pages = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.max_draft = d->max_draft;
  a.out_f32 = d->out_dtype == SD_OUT_F32;
  a.kv_chunk = d->kv_chunk;
  a.v_key_major = d->v_layout == SD_V_KEY_MAJOR;
  a.total_q = total_q;
  a.softmax_scale = d->softmax_scale;
  a.stream = (hipStream_t)stream;
  hipError_t e = sdv_attn_launch(a);
  if (e != hipSuccess) return fail(SD_ERR_HIP, "verify attention launch: %s", hipGetErrorString(e));
  return SD_OK;
}

// The relaxed rule (lossy) adds the JS threshold and the two optional per-row outputs.
struct Relaxed {
  bool on = false;
  float tau = -1.f;
  float* entropy = nullptr;
  float* js = nullptr;
};

sd_status run_accept(const sd_accept_desc* d, int32_t total_q, const float* target, const float* draft,
                     const int32_t* tokens, const int32_t* q_start, const float* uniforms, int32_t* al,
                     int32_t* out_tokens, void* ws, size_t ws_bytes, void* stream, Relaxed rx = Relaxed()) {
  sd_status s = check_accept(d, total_q, rx.on);
  if (s != SD_OK) return s;
  if (rx.on && isnan(rx.tau)) return fail(SD_ERR_INVALID_ARG, "js_threshold is NaN");
  if (d->num_seqs == 0) return SD_OK;
  const bool stoch = d->mode == SD_ACCEPT_STOCHASTIC;
  const bool any_drafts = total_q > d->num_seqs;
  if (!target || !q_start || !al || !out_tokens || (any_drafts && !tokens))
    return fail(SD_ERR_INVALID_ARG, "a required accept pointer is NULL");
  if (stoch && (!uniforms || (any_drafts && !draft)))
    return fail(SD_ERR_INVALID_ARG, "stochastic acceptance needs draft_logits and uniforms");
  if (rx.on && any_drafts && !draft)
    return fail(SD_ERR_INVALID_ARG, "relaxed acceptance needs draft_logits");
  const size_t need = acc_ws(d, total_q, rx.on);
  if (!ws || ws_bytes < need)
    return fail(SD_ERR_WORKSPACE, "accept workspace %zu bytes < required %zu", ws_bytes, need);
  if ((uintptr_t)ws % 16) return fail(SD_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  SdAccLaunch a{};
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.q_start = q_start;
  a.uniforms = uniforms;
  a.accept_len = al;
  a.out_tokens = out_tokens;
  a.workspace = ws;
  a.B = d->num_seqs;
  a.T = total_q;
  a.V = d->vocab;
  a.max_draft = d->max_draft;
  a.stochastic = stoch;
  a.lossy = rx.on;
  a.js_threshold = rx.tau;
  a.out_entropy = rx.entropy;
  a.out_js = rx.js;
  a.stream = (hipStream_t)stream;
  hipError_t e = sdv_accept_launch(a);
  if (e != hipSuccess) return fail(SD_ERR_HIP, "accept/reject launch: %s", hipGetErrorString(e));
  return SD_OK;
}

sd_status check_loop(const sd_loop_desc* d) {
  if (!d) return fail(SD_ERR_INVALID_ARG, "loop descriptor is NULL");
  if (d->num_seqs < 1) return fail(SD_ERR_INVALID_ARG, "num_seqs=%d must be >= 1", d->num_seqs);
  if (d->vocab < 1 || d->vocab > 65536) return fail(SD_ERR_UNSUPPORTED, "vocab=%d must lie in [1, 65536]", d->vocab);
  if (d->max_len < 2) return fail(SD_ERR_INVALID_ARG, "max_len=%d must be >= 2", d->max_len);
  if (d->ngram < 1 || d->ngram > 8) return fail(SD_ERR_UNSUPPORTED, "ngram=%d must lie in [1, 8]", d->ngram);
  if (d->num_tiers < 1 || d->num_tiers > SD_LOOP_MAX_TIERS)
    return fail(SD_ERR_INVALID_ARG, "num_tiers=%d must lie in [1, %d]", d->num_tiers, SD_LOOP_MAX_TIERS);
  for (int t = 0; t < d->num_tiers; ++t) {
    if (d->tiers[t] < 0 || d->tiers[t] > 63) return fail(SD_ERR_UNSUPPORTED, "tier %d = %d must lie in [0, 63]", t, d->tiers[t]);
    if (t > 0 && d->tiers[t] <= d->tiers[t - 1]) return fail(SD_ERR_INVALID_ARG, "tiers must be strictly ascending");
  }
  if (!(d->ema_weight > 0.f && d->ema_weight <= 1.f)) return fail(SD_ERR_INVALID_ARG, "ema_weight must lie in (0, 1]");
  const long long rows = (long long)d->num_seqs * (1 + d->tiers[d->num_tiers - 1]);
  if (rows * ((d->vocab + 1023) / 1024) > 0x7fffffffLL)
    return fail(SD_ERR_UNSUPPORTED, "num_seqs x (1 + largest tier) rows exceed the launch grid");
  return SD_OK;
}

size_t loop_ws(const sd_loop_desc* d) {
  return sdv_loop_workspace_bytes(d->num_seqs, d->vocab, d->num_tiers, d->tiers[d->num_tiers - 1]);
}

sd_status check_gemm(const sd_linear_desc* d) {
  if (!d) return fail(SD_ERR_INVALID_ARG, "linear-layer descriptor is NULL");
  if (d->m < 0) return fail(SD_ERR_INVALID_ARG, "m=%d must be >= 0", d->m);
  if (d->n < 1 || d->k < 1) return fail(SD_ERR_INVALID_ARG, "n=%d and k=%d must be >= 1", d->n, d->k);
  if (d->n % 128 != 0) return fail(SD_ERR_UNSUPPORTED, "n=%d: only multiples of 128 are supported", d->n);
  if (d->k % 64 != 0) return fail(SD_ERR_UNSUPPORTED, "k=%d: only multiples of 64 are supported", d->k);
  if ((long long)d->m * d->n > 0x7fffffffLL || (long long)d->n * d->k > 0x7fffffffLL ||
      (long long)d->m * d->k > 0x7fffffffLL)
    return fail(SD_ERR_UNSUPPORTED, "m*n, n*k and m*k must each be below 2^31");
  return SD_OK;
}

}  // namespace

#define SD_EXPORT __attribute__((visibility("default")))

extern "C" {

SD_EXPORT size_t sd_verify_attention_workspace_size(const sd_attn_desc* desc, int32_t total_q) {
  if (check_attn(desc, total_q) != SD_OK) return 0;
  return attn_ws(desc);
}

SD_EXPORT sd_status sd_verify_attention(const sd_attn_desc* desc, int32_t total_q, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table, const int32_t* kv_len,
                              const int32_t* q_start, void* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return run_attention(desc, total_q, q, k_cache, v_cache, block_table, kv_len, q_start, out, workspace,
                       workspace_bytes, stream);
}

SD_EXPORT size_t sd_accept_reject_workspace_size(const sd_accept_desc* desc, int32_t total_q) {
  if (check_accept(desc, total_q) != SD_OK) return 0;
  return acc_ws(desc, total_q);
}

SD_EXPORT sd_status sd_accept_reject(const sd_accept_desc* desc, int32_t total_q, const float* target_logits,
                           const float* draft_logits, const int32_t* draft_tokens, const int32_t* q_start,
                           const float* uniforms, int32_t* accept_len, int32_t* out_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run_accept(desc, total_q, target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len,
                    out_tokens, workspace, workspace_bytes, stream);
}

SD_EXPORT sd_status sd_accept_reject_noalloc(const sd_accept_desc* desc, int32_t total_q,
                                            const float* target_logits, const float* draft_logits,
                                            const int32_t* draft_tokens, const int32_t* q_start,
                                            const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                                            void* stream) {
  sd_status s = check_accept(desc, total_q);
  if (s != SD_OK) return s;
  const size_t need = acc_ws(desc, total_q);
  const size_t have = sdv_noalloc_scratch_bytes();
  if (need > have)
    return fail(SD_ERR_UNSUPPORTED, "accept/reject needs %zu bytes of scratch, above the %zu the no-allocation "
                "call holds: use sd_accept_reject with a workspace", need, have);
  if (desc->num_seqs == 0) return SD_OK;
  void* ws = nullptr;
  hipError_t e = sdv_noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(SD_ERR_HIP, "no-allocation scratch lookup: %s", hipGetErrorString(e));
  return run_accept(desc, total_q, target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len,
                    out_tokens, ws, have, stream);
}

SD_EXPORT size_t sd_accept_lossy_workspace_size(const sd_accept_desc* desc, int32_t total_q) {
  if (check_accept(desc, total_q, true) != SD_OK) return 0;
  return acc_ws(desc, total_q, true);
}

SD_EXPORT sd_status sd_accept_lossy(const sd_accept_desc* desc, int32_t total_q, const float* target_logits,
                                    const float* draft_logits, const int32_t* draft_tokens, const int32_t* q_start,
                                    const float* uniforms, float js_threshold, int32_t* accept_len,
                                    int32_t* out_tokens, float* draft_entropy, float* js_distance, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Relaxed rx;
  rx.on = true;
  rx.tau = js_threshold;
  rx.entropy = draft_entropy;
  rx.js = js_distance;
  return run_accept(desc, total_q, target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len,
                    out_tokens, workspace, workspace_bytes, stream, rx);
}

SD_EXPORT size_t sd_verify_step_workspace_size(const sd_attn_desc* attn, const sd_accept_desc* acc, int32_t total_q) {
  if (check_attn(attn, total_q) != SD_OK || check_accept(acc, total_q) != SD_OK) return 0;
  if (attn->num_seqs != acc->num_seqs) return 0;
  return align256(attn_ws(attn)) + acc_ws(acc, total_q);
}

SD_EXPORT sd_status sd_verify_step(const sd_attn_desc* attn, const sd_accept_desc* acc, int32_t total_q, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* kv_len, const int32_t* q_start, void* attn_out,
                         const float* target_logits, const float* draft_logits, const int32_t* draft_tokens,
                         const float* uniforms, int32_t* accept_len, int32_t* out_tokens, void* workspace,
                         size_t workspace_bytes, void* stream) {
  sd_status s = check_attn(attn, total_q);
  if (s != SD_OK) return s;
  s = check_accept(acc, total_q);
  if (s != SD_OK) return s;
  if (attn->num_seqs != acc->num_seqs)
    return fail(SD_ERR_INVALID_ARG, "attention num_seqs=%d differs from accept num_seqs=%d", attn->num_seqs,
                acc->num_seqs);
  const size_t a_bytes = align256(attn_ws(attn));
  const size_t need = a_bytes + acc_ws(acc, total_q);
  if (!workspace || workspace_bytes < need)
    return fail(SD_ERR_WORKSPACE, "verify-step workspace %zu bytes < required %zu", workspace_bytes, need);
  s = run_attention(attn, total_q, q, k_cache, v_cache, block_table, kv_len, q_start, attn_out, workspace,
                    a_bytes, stream);
  if (s != SD_OK) return s;
  return run_accept(acc, total_q, target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len,
                    out_tokens, (unsigned char*)workspace + a_bytes, workspace_bytes - a_bytes, stream);
}

SD_EXPORT sd_status sd_verify_tree_attention(const sd_attn_desc* desc, int32_t total_q, const void* q,
                                             const void* k_cache, const void* v_cache, const int32_t* block_table,
                                             const int32_t* kv_len, const int32_t* q_start, const int32_t* parents,
                                             void* out, void* workspace, size_t workspace_bytes, void* stream) {
  sd_status s = check_attn(desc, total_q);
  if (s != SD_OK) return s;
  if (desc->max_draft > 63) return fail(SD_ERR_UNSUPPORTED, "max_draft=%d: a draft tree has at most 64 nodes", desc->max_draft);
  if (desc->num_seqs > 0 && total_q > desc->num_seqs && !parents)
    return fail(SD_ERR_INVALID_ARG, "parents must not be NULL");
  // (without drafts every row is a root, which the causal path computes alike)
  return run_attention(desc, total_q, q, k_cache, v_cache, block_table, kv_len, q_start, out, workspace,
                       workspace_bytes, stream, parents);
}

SD_EXPORT size_t sd_tree_accept_workspace_size(const sd_accept_desc* desc, int32_t total_q) {
  if (check_accept(desc, total_q) != SD_OK || desc->mode != SD_ACCEPT_GREEDY || desc->max_draft > 63) return 0;
  return acc_ws(desc, total_q);
}

SD_EXPORT sd_status sd_tree_accept(const sd_accept_desc* d, int32_t total_q, const float* target_logits,
                                   const int32_t* tree_tokens, const int32_t* q_start, const int32_t* parents,
                                   int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  sd_status s = check_accept(d, total_q);
  if (s != SD_OK) return s;
  if (d->mode != SD_ACCEPT_GREEDY) return fail(SD_ERR_UNSUPPORTED, "draft trees are accepted greedily only");
  if (d->max_draft > 63) return fail(SD_ERR_UNSUPPORTED, "max_draft=%d: a draft tree has at most 64 nodes", d->max_draft);
  if (d->num_seqs == 0) return SD_OK;
  const bool any = total_q > d->num_seqs;
  if (!target_logits || !q_start || !accept_len || !out_tokens || !out_nodes || (any && (!tree_tokens || !parents)))
    return fail(SD_ERR_INVALID_ARG, "a required tree-accept pointer is NULL");
  const size_t need = acc_ws(d, total_q);
  if (!workspace || workspace_bytes < need)
    return fail(SD_ERR_WORKSPACE, "tree-accept workspace %zu bytes < required %zu", workspace_bytes, need);
  if ((uintptr_t)workspace % 16) return fail(SD_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  SdAccLaunch a{};
  a.target = target_logits;
  a.draft = nullptr;
  a.tokens = tree_tokens;
  a.q_start = q_start;
  a.uniforms = nullptr;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.workspace = workspace;
  a.B = d->num_seqs;
  a.T = total_q;
  a.V = d->vocab;
  a.max_draft = d->max_draft;
  a.stochastic = 0;
  a.stream = (hipStream_t)stream;
  hipError_t e = sdv_tree_accept_launch(a, parents, out_nodes);   // (parents is read only for drafted nodes)
  if (e != hipSuccess) return fail(SD_ERR_HIP, "tree accept launch: %s", hipGetErrorString(e));
  return SD_OK;
}

SD_EXPORT size_t sd_closed_loop_workspace_size(const sd_loop_desc* desc) {
  if (check_loop(desc) != SD_OK) return 0;
  return loop_ws(desc);
}

SD_EXPORT sd_status sd_closed_loop(const sd_loop_desc* desc, const float* bigram_logits, int32_t* history,
                                   int32_t* length, int32_t steps, int32_t* accept_trace, int32_t* tier_trace,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  sd_status s = check_loop(desc);
  if (s != SD_OK) return s;
  if (steps < 0) return fail(SD_ERR_INVALID_ARG, "steps=%d must be >= 0", steps);
  if (steps == 0) return SD_OK;
  if (!bigram_logits || !history || !length || !accept_trace || !tier_trace)
    return fail(SD_ERR_INVALID_ARG, "a required closed-loop pointer is NULL");
  const size_t need = loop_ws(desc);
  if (!workspace || workspace_bytes < need)
    return fail(SD_ERR_WORKSPACE, "closed-loop workspace %zu bytes < required %zu", workspace_bytes, need);
  if ((uintptr_t)workspace % 16 || (uintptr_t)bigram_logits % 16)
    return fail(SD_ERR_INVALID_ARG, "bigram_logits and workspace must be 16-byte aligned");
  SdLoopLaunch c{};
  c.W = bigram_logits;
  c.hist = history;
  c.len = length;
  c.al_trace = accept_trace;
  c.tier_trace = tier_trace;
  c.tiers = desc->tiers;
  c.workspace = workspace;
  c.B = desc->num_seqs;
  c.V = desc->vocab;
  c.max_len = desc->max_len;
  c.ngram = desc->ngram;
  c.ntiers = desc->num_tiers;
  c.steps = steps;
  c.use_graphs = desc->use_graphs != 0;
  c.ema_weight = desc->ema_weight;
  c.stream = (hipStream_t)stream;
  hipError_t e = sdv_closed_loop(c);
  if (e != hipSuccess) return fail(SD_ERR_HIP, "closed loop: %s", hipGetErrorString(e));
  return SD_OK;
}

SD_EXPORT size_t sd_verify_linear_workspace_size(const sd_linear_desc* desc) {
  if (check_gemm(desc) != SD_OK) return 0;
  return sdv_gemm_workspace_bytes(desc->m, desc->n, desc->k);
}

SD_EXPORT sd_status sd_verify_linear(const sd_linear_desc* desc, const void* x, const void* w, void* y, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  sd_status s = check_gemm(desc);
  if (s != SD_OK) return s;
  if (desc->m == 0) return SD_OK;
  if (!x || !w || !y) return fail(SD_ERR_INVALID_ARG, "x, w and y must not be NULL");
  if ((uintptr_t)x % 16 || (uintptr_t)w % 16 || (uintptr_t)y % 16 || (uintptr_t)workspace % 16)
    return fail(SD_ERR_INVALID_ARG, "x, w, y and workspace must be 16-byte aligned");
  const size_t need = sdv_gemm_workspace_bytes(desc->m, desc->n, desc->k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SD_ERR_WORKSPACE, "linear-layer workspace %zu bytes < required %zu", workspace_bytes, need);
  SdGemmLaunch a;
  a.x = x;
  a.w = w;
  a.y = y;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.m = desc->m;
  a.n = desc->n;
  a.k = desc->k;
  a.stream = (hipStream_t)stream;
  hipError_t e = sdv_gemm_launch(a);
  if (e != hipSuccess) return fail(SD_ERR_HIP, "verify linear launch: %s", hipGetErrorString(e));
  return SD_OK;
}

SD_EXPORT sd_status sd_validate_inputs(const sd_attn_desc* attn, const sd_accept_desc* acc, int32_t total_q,
                                       const int32_t* block_table, const int32_t* kv_len, const int32_t* q_start,
                                       const int32_t* draft_tokens, const float* uniforms, const float* target_logits,
                                       const float* draft_logits, uint32_t* status_word, void* stream) {
  if (!attn && !acc) return fail(SD_ERR_INVALID_ARG, "sd_validate_inputs needs an attention or an accept descriptor");
  sd_status s = SD_OK;
  if (attn && (s = check_attn(attn, total_q)) != SD_OK) return s;
  if (acc && (s = check_accept(acc, total_q)) != SD_OK) return s;
  if (attn && acc && (attn->num_seqs != acc->num_seqs || attn->max_draft != acc->max_draft))
    return fail(SD_ERR_INVALID_ARG, "the two descriptors disagree on num_seqs or max_draft");
  const int B = attn ? attn->num_seqs : acc->num_seqs;
  if (!status_word || !q_start) return fail(SD_ERR_INVALID_ARG, "status_word and q_start are required");
  if (attn && (!block_table || !kv_len)) return fail(SD_ERR_INVALID_ARG, "block_table and kv_len are required with attn");
  if (acc && total_q > B && !draft_tokens) return fail(SD_ERR_INVALID_ARG, "draft_tokens is required with acc");
  SdValidateLaunch v{};
  v.block_table = attn ? block_table : nullptr;
  v.kv_len = attn ? kv_len : nullptr;
  v.q_start = q_start;
  v.tokens = acc ? draft_tokens : nullptr;
  v.uniforms = acc ? uniforms : nullptr;
  v.target = acc ? target_logits : nullptr;
  v.draft = acc && total_q > B ? draft_logits : nullptr;
  v.status = status_word;
  v.B = B;
  v.T = total_q;
  v.V = acc ? acc->vocab : 1;
  v.max_draft = attn ? attn->max_draft : acc->max_draft;
  v.max_pages = attn ? attn->max_pages_per_seq : 0;
  v.num_pages = attn ? attn->num_pages : 0;
  v.stream = (hipStream_t)stream;
  hipError_t e = sdv_validate_launch(v);
  if (e != hipSuccess) return fail(SD_ERR_HIP, "validation launch: %s", hipGetErrorString(e));
  return SD_OK;
}

SD_EXPORT const char* sd_last_error(void) { return g_error.c_str(); }

SD_EXPORT const char* sd_version(void) { return "sdverify 0.1.0 (gfx950)"; }

}  // extern "C"
