"""Verify attention, fp64 reference — test infrastructure only.

What it computes (the plain definition, row by row):

The translated co-design page ("Draft length and attention performance")
states that the speculated tokens reuse the same KV cache, so each KV head
serves G*(1+D) query rows (G query heads that share one KV head, times the
1+D verify positions).  The verify positions run in one forward pass that
yields a next-token distribution at every position ("How does speculative
decoding speed up LLM inference?", "Mechanism", Verify step), so position i
of the block sees the keys up to and including its own position.

For sequence b with N = kv_len[b] keys (the last 1+D_b of which belong to the
verify block) and verify position i in [0, D_b]:

    P      = N - (1 + D_b) + i              absolute position of row i
    key j  lives at page block_table[b, j // page], slot j % page
    s_j    = scale * <q, k_j>               for j = 0 .. P
    o      = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s)

Query head hq uses KV head hq // G.  scale defaults to 1/sqrt(d).  A row with
P < 0 (a sequence shorter than its own verify block) sees no key and its
output is zero.  bf16 inputs are widened exactly to fp64 here.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> exact float64 values."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _check(q_bits, k_bits, v_bits, block_table, kv_len, q_start, group, v_layout="dim"):
    if q_bits.ndim != 3 or k_bits.ndim != 4 or v_bits.ndim != 4:
        raise ValueError("q [T, Hq, d], k [P, Hkv, page, d], v [P, Hkv, d, page] or [P, Hkv, page, d] expected")
    P, Hkv, ps, d = k_bits.shape
    if v_layout not in ("dim", "key"):
        raise ValueError("v_layout is 'dim' ([P, Hkv, d, page]) or 'key' ([P, Hkv, page, d])")
    if v_bits.shape != ((P, Hkv, d, ps) if v_layout == "dim" else (P, Hkv, ps, d)):
        raise ValueError("v must be [P, Hkv, d, page] (each page stored d-major, v_layout 'dim') "
                         "or [P, Hkv, page, d] (key-major, v_layout 'key')")
    if q_bits.shape[1] != Hkv * group or q_bits.shape[2] != d:
        raise ValueError("q heads must be Hkv*G with the cache's head_dim")
    B = len(kv_len)
    if len(q_start) != B + 1 or block_table.shape[0] != B:
        raise ValueError("q_start [B+1] and block_table [B, pages] expected")
    if q_start[-1] != q_bits.shape[0]:
        raise ValueError("q_start[B] must equal the number of q rows")
    for b in range(B):
        n = int(kv_len[b])
        if n < 0 or n > block_table.shape[1] * ps:
            raise ValueError(f"kv_len[{b}]={n} out of range")
        if q_start[b + 1] - q_start[b] < 1:
            raise ValueError("every sequence has at least one verify row")
        used = block_table[b, : (n + ps - 1) // ps]
        if np.any(used < 0) or np.any(used >= P):
            raise ValueError(f"page id out of range in sequence {b}")


def _sequence_keys(cache_bits, table_row, n, h):
    """Keys 0..n-1 of one sequence and KV head from a [P, Hkv, page, d] cache, in
    position order: [n, d]."""
    ps = cache_bits.shape[2]
    j = np.arange(n)
    pages = table_row[j // ps]
    return bf16_bits_to_f64(cache_bits[pages, h, j % ps, :])


def _sequence_values(cache_bits, table_row, n, h, v_layout="dim"):
    """Values 0..n-1 of one sequence and KV head, in position order: [n, d],
    from a [P, Hkv, d, page] cache (each page stored d-major, v_layout 'dim')
    or a [P, Hkv, page, d] one (key-major like K, v_layout 'key')."""
    if v_layout == "key":
        return _sequence_keys(cache_bits, table_row, n, h)
    ps = cache_bits.shape[3]
    j = np.arange(n)
    pages = table_row[j // ps]
    return bf16_bits_to_f64(cache_bits[pages, h, :, j % ps])


def verify_attention_unit(q_bits, k_bits, v_bits, block_table, kv_len, q_start, group,
                          b: int, h: int, scale: Optional[float] = None, v_layout: str = "dim") -> np.ndarray:
    """Output rows of sequence b, KV head h: float64 [1+D_b, G, d]."""
    d = k_bits.shape[3]
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    n = int(kv_len[b])
    t0 = int(q_start[b])
    rows = int(q_start[b + 1]) - t0            # 1 + D_b
    K = _sequence_keys(k_bits, block_table[b], n, h)
    V = _sequence_values(v_bits, block_table[b], n, h, v_layout)
    out = np.zeros((rows, group, d), dtype=np.float64)
    for i in range(rows):
        P = n - rows + i
        if P < 0:
            continue
        Qg = bf16_bits_to_f64(q_bits[t0 + i, h * group:(h + 1) * group, :])   # [G, d]
        s = scale * (Qg @ K[: P + 1].T)                                      # [G, P+1]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[i] = (w @ V[: P + 1]) / w.sum(axis=1, keepdims=True)
    return out


def verify_attention(q_bits, k_bits, v_bits, block_table, kv_len, q_start, group: int,
                     scale: Optional[float] = None,
                     units: Optional[Iterable[Tuple[int, int]]] = None,
                     workers: int = 1, v_layout: str = "dim") -> np.ndarray:
    """All output rows, float64 [T_q, Hkv*G, d].

    ``units`` restricts the work to the listed (b, h) pairs (other rows are
    NaN); ``workers`` > 1 runs independent units on a thread pool.
    """
    q_bits = np.asarray(q_bits)
    k_bits = np.asarray(k_bits)
    v_bits = np.asarray(v_bits)
    block_table = np.asarray(block_table)
    kv_len = np.asarray(kv_len)
    q_start = np.asarray(q_start)
    _check(q_bits, k_bits, v_bits, block_table, kv_len, q_start, group, v_layout)
    T, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    todo = list(units) if units is not None else [(b, h) for b in range(len(kv_len)) for h in range(Hkv)]

    def run(u):
        b, h = u
        return u, verify_attention_unit(q_bits, k_bits, v_bits, block_table, kv_len, q_start,
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
