"""Pins of the tree-verification oracle against things other than itself.

* a chain (parent of node i is i-1) is the causal verify block: attention and
  greedy acceptance equal the (separately pinned) linear oracles;
* a star (every node's parent is the root): node i attends to the prefix, the
  root and itself, which torch's scaled_dot_product_attention computes in fp64
  on the gathered keys (a library routine);
* acceptance by brute force: every node whose whole root path matches the
  target's top tokens is accepted, and the answer is the deepest (then
  lowest-numbered) of them, found here by enumerating the paths.
"""

import numpy as np
import pytest
import torch

from oracle import accept_greedy, verify_attention
from oracle.attention import _sequence_keys, _sequence_values, bf16_bits_to_f64
from oracle.tree import accept_tree_greedy, tree_ancestors, verify_tree_attention
from tests.oracle_io import attention_args
from workloads import WorkloadSpec, generate


def _spec(**kw):
    base = dict(name="tree_case", batch=3, kv_heads=2, group=2, head_dim=64, kv_len=[200, 90, 150],
                draft_len=[7, 4, 9], vocab=50, mode="greedy", seed=5)
    base.update(kw)
    return WorkloadSpec(**base)


def _random_parents(q_start, rng):
    par = []
    for b in range(len(q_start) - 1):
        T = int(q_start[b + 1] - q_start[b]) - 1
        par += [int(rng.integers(0, i)) for i in range(1, T + 1)]
    return np.asarray(par, np.int32)


def _chain(q_start):
    par = []
    for b in range(len(q_start) - 1):
        T = int(q_start[b + 1] - q_start[b]) - 1
        par += list(range(T))
    return np.asarray(par, np.int32)


def test_chain_tree_is_the_causal_block():
    inp = generate(_spec())
    a = attention_args(inp)
    par = _chain(a["q_start"])
    np.testing.assert_array_equal(verify_tree_attention(parents=par, **a), verify_attention(**a))


def test_star_tree_matches_sdpa_on_gathered_keys():
    inp = generate(_spec(kv_heads=1, group=3))
    a = attention_args(inp)
    qs = a["q_start"]
    par = np.zeros(int(qs[-1]) - (len(qs) - 1), np.int32)
    out = verify_tree_attention(parents=par, **a)
    d = a["k_bits"].shape[3]
    for b in range(len(qs) - 1):
        n = int(a["kv_len"][b])
        t0, t1 = int(qs[b]), int(qs[b + 1])
        T = t1 - t0 - 1
        K = _sequence_keys(a["k_bits"], a["block_table"][b], n, 0)
        V = _sequence_values(a["v_bits"], a["block_table"][b], n, 0, a["v_layout"])
        first = n - 1 - T
        for i in range(T + 1):
            keys = list(range(first + 1)) + ([first + i] if i > 0 else [])
            q = torch.from_numpy(bf16_bits_to_f64(a["q_bits"][t0 + i, 0:3, :]))[:, None, :]   # [G, 1, d]
            k = torch.from_numpy(K[keys])[None].expand(3, -1, -1)
            v = torch.from_numpy(V[keys])[None].expand(3, -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1.0 / np.sqrt(d))
            np.testing.assert_allclose(out[t0 + i, 0:3, :], ref[:, 0, :].numpy(), rtol=0, atol=1e-12)


def test_chain_acceptance_is_linear_greedy():
    rng = np.random.default_rng(3)
    q_start = np.array([0, 5, 6, 14], np.int32)
    V = 7
    target = rng.standard_normal((14, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=11).astype(np.int32)
    # make some leading drafts match
    for b in range(3):
        t0, t1 = q_start[b], q_start[b + 1]
        for i in range(min(2, t1 - t0 - 1)):
            tokens[t0 - b + i] = int(np.argmax(target[t0 + i]))
    al, out, nodes = accept_tree_greedy(target, tokens, q_start, _chain(q_start))
    al2, out2 = accept_greedy(target, tokens, q_start)
    np.testing.assert_array_equal(al, al2)
    np.testing.assert_array_equal(out, out2)
    for b in range(3):
        t0 = q_start[b]
        np.testing.assert_array_equal(nodes[t0:t0 + al[b] - 1], np.arange(1, al[b]))


def _brute_force(target, tokens, q_start, parents):
    B = len(q_start) - 1
    V = target.shape[1]
    res = []
    for b in range(B):
        t0 = int(q_start[b])
        T = int(q_start[b + 1]) - t0 - 1
        d0 = t0 - b
        par = parents[d0:d0 + T]
        best, best_path = 0, []
        for node in range(1, T + 1):
            path = []
            i = node
            while i != 0:
                path.append(i)
                i = int(par[i - 1])
            path.reverse()
            ok = all(0 <= tokens[d0 + c - 1] < V and
                     tokens[d0 + c - 1] == int(np.argmax(target[t0 + (int(par[c - 1]))])) for c in path)
            if ok and (len(path) > len(best_path) or (len(path) == len(best_path) and node < best)):
                best, best_path = node, path
        res.append((best, best_path))
    return res


@pytest.mark.parametrize("seed", range(6))
def test_acceptance_matches_path_enumeration(seed):
    rng = np.random.default_rng(seed)
    B = 4
    sizes = rng.integers(1, 12, size=B)
    q_start = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    V = 4                                     # a small vocabulary makes matches common
    target = rng.standard_normal((int(q_start[-1]), V)).astype(np.float32)
    parents = _random_parents(q_start, rng)
    tokens = rng.integers(0, V, size=len(parents)).astype(np.int32)
    tokens[rng.random(len(tokens)) < 0.1] = V + 3      # some out-of-range drafts
    al, out, nodes = accept_tree_greedy(target, tokens, q_start, parents)
    for b, (best, path) in enumerate(_brute_force(target, tokens, q_start, parents)):
        t0 = int(q_start[b])
        d0 = t0 - b
        assert al[b] == len(path) + 1
        np.testing.assert_array_equal(nodes[t0:t0 + len(path)], path)
        np.testing.assert_array_equal(out[t0:t0 + len(path)], [tokens[d0 + c - 1] for c in path])
        assert out[t0 + len(path)] == int(np.argmax(target[t0 + best]))
        assert np.all(out[t0 + al[b]:int(q_start[b + 1])] == -1)


def test_parents_must_precede_children():
    with pytest.raises(ValueError):
        tree_ancestors([0, 2])
    assert tree_ancestors([0, 0, 1]) == [{0}, {0, 1}, {0, 2}, {0, 1, 3}]


def test_tree_workload_shape():
    """The tree drafter of workloads/: a full tree in level order (parents
    precede children), distinct sibling tokens, the same shape per sequence."""
    from workloads import WorkloadSpec, tree_inputs, tree_parents
    par = tree_parents([2, 2, 2, 2])
    assert len(par) == 30 and all(0 <= p < i for i, p in enumerate(par, start=1))
    assert [par.count(p) for p in range(15)] == [2] * 15
    sp = WorkloadSpec(name="t", batch=2, kv_heads=1, group=2, head_dim=64, kv_len=100, draft_len=1, vocab=50,
                      mode="greedy", target_std=3.0, draft_noise_std=1.0)
    inp, parents, tokens = tree_inputs(sp, [3, 2])
    assert inp.q.shape[0] == 2 * 10 and parents.tolist() == tree_parents([3, 2]) * 2
    for b in range(2):
        tk = tokens[b * 9:(b + 1) * 9].tolist()
        for p in range(10):
            sib = [tk[i - 1] for i, q in enumerate(tree_parents([3, 2]), start=1) if q == p]
            assert len(set(sib)) == len(sib)
