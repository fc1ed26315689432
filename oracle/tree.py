"""Tree verification, fp64 reference — test infrastructure only.

The drafted continuations can form a tree instead of one chain: candidate
tokens from several draft heads are combined into a tree of possible
continuations, the target evaluates the whole tree in one forward pass with
tree attention (an attention mask that keeps the causal order inside each
branch), and, as with a chain, the longest accepted candidate prefix moves on
to the next step (the LLM inference handbook, section "Medusa").

Layout (the rows of the linear verify block): sequence b has 1+T_b tree nodes
at verify rows q_start[b] .. q_start[b+1]-1.  Node 0 is the root (the last
emitted token); nodes 1..T_b are drafted tokens, numbered so that every parent
comes before its children: parents[(q_start[b]-b) + i-1] is the parent of node
i, in [0, i), and tree_tokens at the same index is node i's token.  The nodes'
keys and values are the last 1+T_b positions of the sequence's cache, in node
order.

Attention: node i attends to the prefix keys 0 .. N-2-T_b and to the keys of
the nodes on its root path (its ancestors and itself).  A chain (parent of i =
i-1) is the causal verify block.

Greedy acceptance: the root is accepted; node c is accepted iff its parent p
is, and its token lies in [0, V) and equals the target's top token at row p
(lowest index on ties).  The accepted node of largest depth (the smallest node
index among equal depths) ends the accepted path: AL = its depth + 1, and the
emitted tokens are the tokens of the path's nodes followed by the target's top
token at that node.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, List, Optional, Set, Tuple

import numpy as np

from .attention import _check, _sequence_keys, _sequence_values, bf16_bits_to_f64


def _seq(q_start, b):
    t0 = int(q_start[b])
    T = int(q_start[b + 1]) - t0 - 1
    return t0, T, t0 - b


def tree_ancestors(parents_b) -> List[Set[int]]:
    """For a tree of 1+T nodes given by parents_b[i-1] = parent of node i:
    the set of nodes on each node's root path (itself included)."""
    anc = [{0}]
    for i in range(1, len(parents_b) + 1):
        p = int(parents_b[i - 1])
        if not 0 <= p < i:
            raise ValueError(f"parent of node {i} is {p}: parents must precede their children")
        anc.append(anc[p] | {i})
    return anc


def verify_tree_attention_unit(q_bits, k_bits, v_bits, block_table, kv_len, q_start, parents, group,
                               b: int, h: int, scale: Optional[float] = None, v_layout: str = "dim") -> np.ndarray:
    """Output rows of sequence b, KV head h under the tree mask: float64 [1+T_b, G, d]."""
    d = k_bits.shape[3]
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    n = int(kv_len[b])
    t0, T, d0 = _seq(q_start, b)
    anc = tree_ancestors(np.asarray(parents)[d0:d0 + T])
    K = _sequence_keys(k_bits, block_table[b], n, h)
    V = _sequence_values(v_bits, block_table[b], n, h, v_layout)
    first = n - 1 - T                          # key position of the root
    out = np.zeros((1 + T, group, d), dtype=np.float64)
    for i in range(1 + T):
        keys = [j for j in range(max(first, 0))] + sorted(first + a for a in anc[i] if first + a >= 0)
        if not keys:
            continue
        Qg = bf16_bits_to_f64(q_bits[t0 + i, h * group:(h + 1) * group, :])
        s = scale * (Qg @ K[keys].T)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[i] = (w @ V[keys]) / w.sum(axis=1, keepdims=True)
    return out


def verify_tree_attention(q_bits, k_bits, v_bits, block_table, kv_len, q_start, parents, group: int,
                          scale: Optional[float] = None, units: Optional[Iterable[Tuple[int, int]]] = None,
                          workers: int = 1, v_layout: str = "dim") -> np.ndarray:
    """All output rows under the tree mask, float64 [T_q, Hkv*G, d] (rows of
    units not listed in ``units`` are NaN)."""
    q_bits, k_bits, v_bits = np.asarray(q_bits), np.asarray(k_bits), np.asarray(v_bits)
    block_table, kv_len, q_start = np.asarray(block_table), np.asarray(kv_len), np.asarray(q_start)
    _check(q_bits, k_bits, v_bits, block_table, kv_len, q_start, group, v_layout)
    T, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    todo = list(units) if units is not None else [(b, h) for b in range(len(kv_len)) for h in range(Hkv)]

    def run(u):
        b, h = u
        return u, verify_tree_attention_unit(q_bits, k_bits, v_bits, block_table, kv_len, q_start, parents,
                                             group, b, h, scale, v_layout)

    if workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(run, todo))
    else:
        results = [run(u) for u in todo]
    for (b, h), o in results:
        t0, t1 = int(q_start[b]), int(q_start[b + 1])
        out[t0:t1, h * group:(h + 1) * group, :] = o
    return out


def accept_tree_greedy(target_logits, tree_tokens, q_start, parents):
    """Greedy acceptance along the tree.  Returns (accept_len [B], out_tokens
    [T_q], out_nodes [T_q]): out_tokens[t0+k] for k < AL (the path's tokens,
    then the target's top token at its last node), out_nodes[t0+k] for
    k < AL-1 (the path's node indices, 1..T_b), -1 elsewhere."""
    target = np.asarray(target_logits, dtype=np.float32)
    tokens = np.asarray(tree_tokens)
    parents = np.asarray(parents)
    q_start = np.asarray(q_start)
    B = len(q_start) - 1
    V = target.shape[1]
    al = np.zeros(B, dtype=np.int32)
    out = np.full(target.shape[0], -1, dtype=np.int32)
    nodes = np.full(target.shape[0], -1, dtype=np.int32)
    for b in range(B):
        t0, T, d0 = _seq(q_start, b)
        par = [int(p) for p in parents[d0:d0 + T]]
        tree_ancestors(par)                    # validates the order
        top = [int(np.argmax(target[t0 + i])) for i in range(1 + T)]   # first maximum = lowest id
        accepted = [True] + [False] * T
        depth = [0] * (1 + T)
        best = 0
        for i in range(1, 1 + T):
            p = par[i - 1]
            x = int(tokens[d0 + i - 1])
            depth[i] = depth[p] + 1
            accepted[i] = accepted[p] and 0 <= x < V and x == top[p]
            if accepted[i] and depth[i] > depth[best]:
                best = i
        path = []
        i = best
        while i != 0:
            path.append(i)
            i = par[i - 1]
        path.reverse()
        for k, node in enumerate(path):
            out[t0 + k] = int(tokens[d0 + node - 1])
            nodes[t0 + k] = node
        out[t0 + len(path)] = top[best]
        al[b] = len(path) + 1
    return al, out, nodes
