"""CPU oracle of the speculative-decoding verify step — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 statement of what the verify step computes, written from
the pages' definitions:

* attention.py — the (1+D) verify positions of each sequence attend over the
  sequence's KV cache under a causal mask, G query heads per KV head
  ("Co-Designing AI Models Using Speculative Decoding for Faster LLM
  Inference", translated page, section "Draft length and attention
  performance").
* accept.py — greedy first-mismatch acceptance, and min(1, p/q) acceptance
  with residual resampling plus the extra target token ("How does speculative
  decoding speed up LLM inference?", sections "Mechanism" and "Math
  intuition"; the NVIDIA page's "What is speculative decoding?" for D and AL;
  the LLM inference handbook's "How speculative decoding works").
* tree.py — tree verification: attention under the ancestor mask of a draft
  tree, and greedy acceptance of its longest accepted path (the LLM inference
  handbook, section "Medusa").
* lossy.py — acceptance relaxed by the Jensen-Shannon distance between the
  draft and target distributions, with the draft entropy reported per row
  (the LLM inference handbook, section "AdaSD").
* loop.py — a closed speculative-decoding loop on a bigram toy LM: an n-gram
  drafter, greedy verification and an EMA-of-AL controller over draft-length
  tiers (the LLM inference handbook, section on SGLang's adaptive speculative
  decoding).
* gemm.py — the verify-shaped linear layer y = x W^T whose GEMM-M grows to
  M*(1+D) under speculation (the co-design page, section "Draft length and
  performance of linear layers").

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
or call anything here.  The product path (the HIP library and its Python
binding) never does, and this package imports nothing from it: the two share
only the seeded input generators in ``workloads/``.
"""

from .attention import bf16_bits_to_f64, verify_attention, verify_attention_unit
from .accept import accept_greedy, accept_stochastic, accept_reject, row_log_normalizer
from .gemm import linear_abs_sum, verify_linear
from .lossy import accept_lossy, js_distance, row_entropy
from .tree import accept_tree_greedy, tree_ancestors, verify_tree_attention, verify_tree_attention_unit

__all__ = [
    "bf16_bits_to_f64", "verify_attention", "verify_attention_unit",
    "accept_greedy", "accept_stochastic", "accept_reject", "row_log_normalizer",
    "verify_linear", "linear_abs_sum", "accept_lossy", "js_distance", "row_entropy",
    "verify_tree_attention", "verify_tree_attention_unit", "accept_tree_greedy", "tree_ancestors",
]
