/*
 * sd_verify.h — the target-model verify step of speculative decoding on
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The verify step has two parts:
 *
 *  1. Verify attention.  The 1+D_b positions of sequence b (the last emitted
 *     token followed by D_b drafted tokens) attend over the sequence's paged
 *     KV cache in one pass.  The speculated tokens reuse the same KV cache, so
 *     each KV head serves G*(1+D_b) query rows ("Co-Designing AI Models Using
 *     Speculative Decoding for Faster LLM Inference", translated page, section
 *     "Draft length and attention performance").  Every verify position yields
 *     its own next-token distribution in that pass ("How does speculative
 *     decoding speed up LLM inference?", section "Mechanism", Verify step), so
 *     position i sees keys up to its own position (a causal mask inside the
 *     block).
 *
 *  2. Accept / reject over the vocabulary.  Greedy: accept drafts until the
 *     first mismatch with the target's top token (the co-design page, "What is
 *     speculative decoding?").  Stochastic: accept draft x with probability
 *     min(1, p(x)/q(x)); at the first rejection resample from the normalised
 *     residual max(0, p - q) ("How does speculative decoding speed up LLM
 *     inference?", sections "Mechanism" and "Math intuition").  The target
 *     always yields one more token, so the acceptance length AL is in
 *     [1, 1+D_b] (the co-design page, "What is speculative decoding?").
 *
 * Conventions for every call:
 *  - All array arguments are DEVICE pointers, allocated and owned by the
 *    caller.  The library never allocates, frees or synchronises; each call
 *    enqueues its kernels on `stream` (a hipStream_t, NULL = default stream)
 *    and returns.  Outputs are valid once that stream has reached them.
 *  - Host-checkable preconditions (sizes, supported shapes, non-NULL pointers,
 *    workspace size) are validated before anything is enqueued; a violation
 *    returns a non-zero sd_status, enqueues nothing, and sd_last_error()
 *    describes it.  Nothing is thrown and nothing aborts across this ABI.
 *  - Device-side contents are the caller's contract: page ids in range for
 *    the pages a sequence uses, kv_len[b] <= max_pages_per_seq*page_size,
 *    q_start non-decreasing with q_start[B] == total_q, finite or -inf
 *    logits (no row entirely -inf), uniforms in [0, 1).  Kernels clamp
 *    indices so that a violation cannot read or write out of bounds; the
 *    values computed for an offending sequence are then unspecified.
 *    sd_validate_inputs checks this contract on request.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - Concurrent calls are safe when they use distinct workspaces and outputs.
 *
 * Sequence layout shared by both parts: sequence b owns the verify rows
 * q_start[b] .. q_start[b+1]-1 (1+D_b rows, D_b >= 0); row q_start[b]+i is
 * verify position i.  Its D_b draft rows and drafted tokens sit at
 * (q_start[b]-b)+i, i < D_b (so there are T_d = total_q - B of them).
 */
#ifndef SD_VERIFY_H
#define SD_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SD_OK = 0,
  SD_ERR_INVALID_ARG = 1,   /* a host-side precondition failed */
  SD_ERR_UNSUPPORTED = 2,   /* valid request outside the built kernel variants */
  SD_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than the *_workspace_size query */
  SD_ERR_HIP = 4            /* the HIP runtime reported an error while enqueueing */
} sd_status;

typedef enum { SD_ACCEPT_GREEDY = 0, SD_ACCEPT_STOCHASTIC = 1 } sd_accept_mode;
typedef enum { SD_OUT_BF16 = 0, SD_OUT_F32 = 1 } sd_out_dtype;

/* How each (page, head) block of the V cache is stored.  SD_V_KEY_MAJOR:
 * [page_size][d] like K (the usual paged cache); SD_V_DIM_MAJOR: [d][page_size]
 * (the transpose), which the kernels read with plain 16-byte LDS loads where
 * key-major pages need transposing ones. */
typedef enum { SD_V_KEY_MAJOR = 0, SD_V_DIM_MAJOR = 1 } sd_v_layout;

/* Verify-attention problem description (host memory, read during the call). */
typedef struct {
  int32_t num_seqs;           /* B >= 0 */
  int32_t num_kv_heads;       /* H_kv >= 1 */
  int32_t group_size;         /* G >= 1: query heads per KV head; query head hq uses KV head hq / G */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t page_size;          /* keys per page: 16 */
  int32_t max_pages_per_seq;  /* columns of block_table */
  int32_t num_pages;          /* pages in each of the K and V pools */
  int32_t max_draft;          /* upper bound on every D_b; G*(1+max_draft) <= 256 */
  float softmax_scale;        /* scores are scale * q.k; 0 selects 1/sqrt(d) */
  int32_t out_dtype;          /* sd_out_dtype */
  int32_t kv_chunk;           /* keys per split-KV work item: a multiple of 64, at most 8192; 0 = chosen per call */
  int32_t v_layout;           /* sd_v_layout of v_cache */
} sd_attn_desc;

/* Accept/reject problem description. */
typedef struct {
  int32_t num_seqs;           /* B >= 0 */
  int32_t vocab;              /* V >= 1 */
  int32_t max_draft;          /* upper bound on every D_b */
  int32_t mode;               /* sd_accept_mode */
} sd_accept_desc;

/*
 * Workspace bytes sd_verify_attention needs for this description and
 * total_q = sum_b (1+D_b) verify rows.  Returns 0 for an invalid description.
 * The size does not depend on the KV lengths: the split of the keys into work
 * items is planned on the device at every call, within an item budget fixed
 * by B, H_kv and the GPU's compute-unit count, so one workspace serves every
 * call of the same shape however the caches grow.  total_q is an argument of
 * the calls too, so that the host can check the row count against the
 * workspace without reading q_start from the device.
 */
size_t sd_verify_attention_workspace_size(const sd_attn_desc* desc, int32_t total_q);

/*
 * Verify attention.  For sequence b with N = kv_len[b] keys, of which the
 * last 1+D_b are its own verify positions, row i (absolute position
 * P = N-(1+D_b)+i) of query head hq attends to keys 0..P of KV head hq/G:
 *     o = sum_j softmax_j(scale * q.k_j) v_j,
 * with key j stored at page block_table[b*max_pages_per_seq + j/page_size],
 * slot j % page_size.  A row with P < 0 sees no key and its output is zero.
 *
 *   q            bf16 [total_q, H_kv*G, d]                 row-major
 *   k_cache      bf16 [num_pages, H_kv, page_size, d]      row-major
 *   v_cache      bf16 [num_pages, H_kv, page_size, d]      row-major, desc->v_layout = SD_V_KEY_MAJOR;
 *                bf16 [num_pages, H_kv, d, page_size]      with SD_V_DIM_MAJOR (each page's block
 *                stored transposed, so that the keys a P.V product contracts over
 *                are contiguous)
 *   block_table  int32 [B, max_pages_per_seq]
 *   kv_len       int32 [B]
 *   q_start      int32 [B+1]
 *   out          [total_q, H_kv*G, d], bf16 or fp32 per desc->out_dtype; written, not read
 *   workspace    device scratch of at least sd_verify_attention_workspace_size bytes,
 *                16-byte aligned; its contents on entry do not matter
 *
 * Scores, softmax and accumulation are fp32; bf16 output is rounded to
 * nearest-even.
 */
sd_status sd_verify_attention(const sd_attn_desc* desc, int32_t total_q,
                              const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* kv_len,
                              const int32_t* q_start, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sd_accept_reject needs.  Returns 0 for an invalid description. */
size_t sd_accept_reject_workspace_size(const sd_accept_desc* desc, int32_t total_q);

/*
 * Accept / reject.  For sequence b with t0 = q_start[b], D = q_start[b+1]-t0-1
 * and draft base d0 = t0 - b:
 *   target row t0+i (i = 0..D) holds the target's logits after position i;
 *   draft row d0+i (i < D) holds the logits draft_tokens[d0+i] = x_{i+1} was drawn from.
 *
 * Greedy (draft_logits and uniforms may be NULL): x_{i+1} passes iff it equals
 *   the lowest-index maximum of target row t0+i (compared as fp32).
 * Stochastic: with p = softmax(target row), q = softmax(draft row), x passes
 *   iff (double)uniforms[t0+i] < exp((log p(x)) - (log q(x))), evaluated in
 *   fp64 from the fp32 logits (q(x)=0<p(x) passes; p(x)=0 fails).
 * In both modes a token outside [0, V) fails.  With n the number of leading
 * passes: accept_len[b] = n+1; out_tokens[t0+k] = x_{k+1} for k < n; then
 *   greedy:      out_tokens[t0+n] = the target's top token at row n;
 *   stochastic:  out_tokens[t0+n] = smallest j with C_j > uniforms[t0+D] * Z,
 *                where C is the inclusive prefix sum over ascending token ids of
 *                w = max(0, p - q) at row n if n < D, else w = p at row D, and
 *                Z = C_{V-1} (w = p if the residual sums to zero);
 *   out_tokens[t0+k] = -1 for n < k <= D.
 *
 *   target_logits fp32 [total_q, V];  draft_logits fp32 [total_q - B, V]
 *   draft_tokens int32 [total_q - B]; q_start int32 [B+1]; uniforms fp32 [total_q]
 *   accept_len int32 [B] (written);  out_tokens int32 [total_q] (written)
 *
 * Row sums of exponentials are accumulated in fp64; the tests, the residual
 * and the inverse-CDF scan are evaluated in fp64.
 */
sd_status sd_accept_reject(const sd_accept_desc* desc, int32_t total_q,
                           const float* target_logits, const float* draft_logits,
                           const int32_t* draft_tokens, const int32_t* q_start,
                           const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Accept / reject with no workspace argument, for callers that cannot
 * allocate device memory themselves (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and errors as sd_accept_reject without the workspace: the call uses scratch
 * the library holds in a static device array of SD_NOALLOC_SCRATCH_BYTES per
 * GPU (kept until the process ends) and allocates nothing.  A problem whose
 * sd_accept_reject_workspace_size exceeds that returns SD_ERR_UNSUPPORTED and
 * enqueues nothing.  Every call on one GPU shares that GPU's array: calls
 * whose kernels may overlap on one GPU (different streams, or different host
 * threads without ordering) race on it, so the caller orders them.
 */
#define SD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
sd_status sd_accept_reject_noalloc(const sd_accept_desc* desc, int32_t total_q,
                                   const float* target_logits, const float* draft_logits,
                                   const int32_t* draft_tokens, const int32_t* q_start,
                                   const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                                   void* stream);

/* Workspace bytes sd_accept_lossy needs.  Returns 0 for an invalid description. */
size_t sd_accept_lossy_workspace_size(const sd_accept_desc* desc, int32_t total_q);

/*
 * Relaxed (lossy) accept / reject.  Adaptive speculative decoding may loosen
 * how strictly each draft token is checked, so that tokens close enough to the
 * target pass and the output leaves the target's exact distribution; AdaSD
 * decides "close enough" by the Jensen-Shannon distance between the draft and
 * target distributions and reports the draft entropy, which tells the drafter
 * when to stop (the LLM inference handbook, sections on adaptive speculative
 * decoding and "AdaSD").
 *
 * As sd_accept_reject (same layouts, modes and sampling after the first
 * failure), except that draft x_{i+1} of a sequence also passes when
 *   JS(p_i, q_i) <= js_threshold,
 * with p_i = softmax(target row t0+i), q_i = softmax(draft row d0+i) and
 * JS = sqrt(KL(p||m)/2 + KL(q||m)/2), m = (p+q)/2, natural logarithms
 * (0 <= JS <= sqrt(ln 2)).  A token outside [0, V) never passes.  A negative
 * js_threshold gives the lossless result; NaN is rejected.  draft_logits are
 * required in both modes (uniforms only for SD_ACCEPT_STOCHASTIC).
 *
 *   draft_entropy fp32 [total_q - B] or NULL: -sum_j q_i(j) ln q_i(j) of every
 *                 drafted row, written also past the first failure;
 *   js_distance   fp32 [total_q - B] or NULL: JS(p_i, q_i) of every drafted row.
 *
 * The divergence terms are evaluated in fp32 per token and summed in fp64;
 * the statistics and the threshold test are taken in fp64 from those sums.
 * Extra cost over sd_accept_reject: one more read of every drafted target and
 * draft row.
 */
sd_status sd_accept_lossy(const sd_accept_desc* desc, int32_t total_q,
                          const float* target_logits, const float* draft_logits,
                          const int32_t* draft_tokens, const int32_t* q_start,
                          const float* uniforms, float js_threshold,
                          int32_t* accept_len, int32_t* out_tokens,
                          float* draft_entropy, float* js_distance,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for sd_verify_step: one buffer holding both parts' scratch. */
size_t sd_verify_step_workspace_size(const sd_attn_desc* attn, const sd_accept_desc* acc,
                                     int32_t total_q);

/*
 * One verify step: the target scores all 1+D_b positions of every sequence in
 * one pass and the drafts are accepted or rejected against those scores in
 * the same step ("How does speculative decoding speed up LLM inference?",
 * section "Mechanism", Verify step).  Here: sd_verify_attention followed by
 * sd_accept_reject on the same stream, sharing one workspace (the target
 * logits come from the caller's LM head between the two in a full model;
 * the call takes them as an input).  attn->num_seqs must equal
 * acc->num_seqs; arguments are as in the two calls above.
 */
sd_status sd_verify_step(const sd_attn_desc* attn, const sd_accept_desc* acc, int32_t total_q,
                         const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* kv_len, const int32_t* q_start,
                         void* attn_out,
                         const float* target_logits, const float* draft_logits,
                         const int32_t* draft_tokens, const float* uniforms,
                         int32_t* accept_len, int32_t* out_tokens,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tree verification (an extension next to the verify step proper).  The drafts
 * of a sequence may form a tree instead of one chain: the target scores the
 * whole tree in one pass with an attention mask that keeps the causal order
 * inside each branch, and the longest accepted candidate prefix moves on (the
 * LLM inference handbook, section "Medusa").
 *
 * Layout, as for the linear block: sequence b has 1+T_b tree nodes at verify
 * rows q_start[b] .. q_start[b+1]-1, node 0 being the root (the last emitted
 * token) and nodes 1..T_b drafted tokens, numbered so that every parent comes
 * before its children.  With d0 = q_start[b]-b, parents[d0+i-1] in [0, i) is
 * the parent of node i and tree_tokens[d0+i-1] its token.  The nodes' keys and
 * values are the last 1+T_b positions of the sequence's cache, in node order.
 */

/*
 * Attention under the tree mask: node i attends to the keys before the tree
 * and to the nodes on its root path (its ancestors and itself); otherwise as
 * sd_verify_attention, with the same workspace size query.  At most 64 nodes
 * per tree (desc->max_draft <= 63).  A parent outside [0, i) is taken as the
 * root.  parents int32 [total_q - B] (may be NULL when total_q == B).
 */
sd_status sd_verify_tree_attention(const sd_attn_desc* desc, int32_t total_q,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* kv_len,
                                   const int32_t* q_start, const int32_t* parents, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sd_tree_accept needs (desc->mode must be SD_ACCEPT_GREEDY, desc->max_draft <= 63); 0 if invalid. */
size_t sd_tree_accept_workspace_size(const sd_accept_desc* desc, int32_t total_q);

/*
 * Greedy acceptance of a draft tree.  The root is accepted; node c is accepted
 * iff its parent p is, and its token lies in [0, V) and equals the lowest-index
 * maximum of target row q_start[b]+p.  The accepted node of largest depth (the
 * lowest index among equal depths) ends the path of L nodes below the root:
 *   accept_len[b] = L+1;
 *   out_tokens[t0+k] = the token of the path's node at depth k+1 (k < L),
 *   out_tokens[t0+L] = the target's top token at the path's last node,
 *   out_nodes[t0+k] = the index of the path's node at depth k+1 (k < L);
 * other entries up to t0+T_b are -1.  A parent outside [0, i) is taken as the
 * root.  desc->mode must be SD_ACCEPT_GREEDY, and a tree has at most 64 nodes
 * (desc->max_draft <= 63); SD_ERR_UNSUPPORTED otherwise.
 *
 *   target_logits fp32 [total_q, V];  tree_tokens, parents int32 [total_q - B]
 *   accept_len int32 [B]; out_tokens, out_nodes int32 [total_q] (written)
 */
sd_status sd_tree_accept(const sd_accept_desc* desc, int32_t total_q, const float* target_logits,
                         const int32_t* tree_tokens, const int32_t* q_start, const int32_t* parents,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Closed speculative-decoding loop on a toy LM (an extension next to the
 * verify step proper).  Each round drafts D tokens per sequence, verifies them
 * in one pass and keeps the accepted prefix; after each round the mean
 * acceptance length feeds an exponential moving average (EMA) that picks the
 * next round's D among a few tiers, each tier with its own captured HIP graph,
 * so that switching tiers costs no recapture (the LLM inference handbook,
 * section on SGLang's adaptive speculative decoding, default tiers [1, 3, 7]).
 * Only the speculation length adapts, so the output is the target's greedy
 * decoding.
 *
 *   target    a bigram toy LM: the logits after token a are row a of
 *             bigram_logits (fp32 [V, V]); verification is sd_accept_reject's
 *             greedy rule;
 *   drafter   model-free n-gram lookup: the latest earlier occurrence of the
 *             history's last k tokens (k = ngram, ngram-1, ..., 1) proposes the
 *             D tokens that followed it (-1, never accepted, where the history
 *             ends or nothing matches);
 *   controller ema starts at 1; after round s, ema = (1-w) ema + w mean(AL)
 *             over the sequences that appended; the next D is the smallest
 *             tier >= ema, else the largest tier.
 *
 * history int32 [B, max_len] and length int32 [B] (device; length >= 1) are
 * updated in place: a round appends the AL emitted tokens of each sequence,
 * or nothing once they would pass max_len.  accept_trace int32 [steps, B] and
 * tier_trace int32 [steps] are host buffers (pinned memory is fastest) that
 * receive the tokens appended per sequence and the D of each round.
 *
 * Unlike the other calls this one waits for the stream once per round (to
 * read the acceptance lengths), and with use_graphs != 0 it creates a
 * non-blocking capture stream and one graph per tier, and destroys all of
 * them before it returns (it allocates no device memory).  tiers: 1..8 strictly ascending values in
 * [0, 63]; ngram in [1, 8]; vocab <= 65536; ema_weight in (0, 1].
 */
#define SD_LOOP_MAX_TIERS 8
typedef struct {
  int32_t num_seqs;                    /* B >= 1 */
  int32_t vocab;                       /* V */
  int32_t max_len;                     /* history capacity per sequence */
  int32_t ngram;                       /* drafter order */
  int32_t num_tiers;
  int32_t tiers[SD_LOOP_MAX_TIERS];    /* draft lengths, ascending */
  float ema_weight;                    /* w */
  int32_t use_graphs;                  /* 1: one captured graph per tier; 0: direct launches */
} sd_loop_desc;

size_t sd_closed_loop_workspace_size(const sd_loop_desc* desc);

sd_status sd_closed_loop(const sd_loop_desc* desc, const float* bigram_logits,
                         int32_t* history, int32_t* length, int32_t steps,
                         int32_t* accept_trace, int32_t* tier_trace,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Verify-shaped linear layer (an extension next to the verify step proper).
 * With speculation every linear layer of the target sees M*(1+D) rows in the
 * verify pass instead of M, against the same weight: the GEMM-M grows by the
 * factor 1+D while the bytes of W stay the same ("Co-Designing AI Models Using
 * Speculative Decoding for Faster LLM Inference", translated page, section
 * "Draft length and performance of linear layers", Figure 3, for an expert
 * GEMM of N = K = 6144).
 */
typedef struct {
  int32_t m;   /* rows of x and y (the verify rows, M*(1+D)), >= 0 */
  int32_t n;   /* output features (rows of W): a positive multiple of 128 */
  int32_t k;   /* input features: a positive multiple of 64; m*n, n*k, m*k < 2^31 */
} sd_linear_desc;

/* Workspace bytes sd_verify_linear needs (0 is a valid answer: then workspace may be NULL). */
size_t sd_verify_linear_workspace_size(const sd_linear_desc* desc);

/*
 * y = x W^T:  y[m][n] = sum_k x[m][k] * w[n][k], fp32 accumulation, bf16 output
 * rounded to nearest-even.
 *
 *   x          bf16 [m, k]   row-major
 *   w          bf16 [n, k]   row-major (one row per output feature)
 *   y          bf16 [m, n]   row-major; written, not read
 *   workspace  device scratch of at least sd_verify_linear_workspace_size bytes, 16-byte
 *              aligned (fp32 partial sums when K is split); its contents on entry do not matter
 *
 * Deterministic: partial sums over K ranges are added in a fixed order.
 */
sd_status sd_verify_linear(const sd_linear_desc* desc, const void* x, const void* w, void* y,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Opt-in check of the device-side contract above (the verify calls do not
 * check it: they clamp what they index, and a violating sequence gets
 * unspecified values).  One pass over the given inputs; *status_word (one
 * device uint32, overwritten) becomes the OR of the SD_BAD_* bits of every
 * violation found, 0 when there is none.  Either descriptor may be NULL to
 * check one half only (both given: num_seqs and max_draft must agree):
 *  - always: q_start [B+1] (SD_BAD_Q_START);
 *  - with attn: kv_len [B] against each sequence's 1+D_b rows and
 *    max_pages_per_seq*page_size keys (SD_BAD_KV_LEN), and the first
 *    ceil(kv_len[b]/page_size) entries of block_table row b (SD_BAD_PAGE);
 *  - with acc: draft_tokens [total_q - B] (SD_BAD_TOKEN), uniforms [total_q]
 *    when not NULL (SD_BAD_UNIFORM), and target_logits [total_q, V] and
 *    draft_logits [total_q - B, V] when not NULL (SD_BAD_LOGITS; a full pass
 *    over the logits).
 * Every index the pass reads is range-checked first, so it stays in bounds
 * on any input.  Stream-ordered like the other calls; read the word after
 * the stream has reached it.
 */
typedef enum {
  SD_BAD_Q_START = 1,   /* q_start[0] != 0, a sequence with no row or more than 1+max_draft, q_start[B] != total_q */
  SD_BAD_KV_LEN = 2,    /* kv_len[b] < 1+D_b, or > max_pages_per_seq*page_size */
  SD_BAD_PAGE = 4,      /* a page id a sequence uses outside [0, num_pages) */
  SD_BAD_TOKEN = 8,     /* a drafted token outside [0, vocab) */
  SD_BAD_UNIFORM = 16,  /* a uniform outside [0, 1), NaN included */
  SD_BAD_LOGITS = 32    /* a NaN or +inf logit, or a row with every logit -inf */
} sd_bad_input;

sd_status sd_validate_inputs(const sd_attn_desc* attn, const sd_accept_desc* acc, int32_t total_q,
                             const int32_t* block_table, const int32_t* kv_len, const int32_t* q_start,
                             const int32_t* draft_tokens, const float* uniforms, const float* target_logits,
                             const float* draft_logits, uint32_t* status_word, void* stream);

/* Message describing the last non-OK status returned on the calling thread. */
const char* sd_last_error(void);

/* Library version string. */
const char* sd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SD_VERIFY_H */
