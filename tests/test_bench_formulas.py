"""bench.py's algorithmic byte and flop counts, checked against brute-force
counts on small workloads (the roofline figures rest on them), and the
one-GPU contract of its command line."""

import subprocess
import sys

import numpy as np

import bench
from workloads import WorkloadSpec, generate
from workloads.tree import tree_inputs


def _spec(**kw):
    base = dict(name="formula_case", batch=3, kv_heads=2, group=4, head_dim=64, kv_len=[40, 17, 100],
                draft_len=[3, 0, 7], vocab=50, mode="stochastic")
    base.update(kw)
    return WorkloadSpec(**base)


def test_attention_bytes_and_flops_by_brute_force():
    inp = generate(_spec())
    nbytes, flops = bench.algorithmic_attention(inp)
    kv = inp.kv_len.numpy()
    qs = inp.q_start.numpy()
    sp = inp.spec
    # count every (query row, visible key) pair one by one: row i of sequence b sees keys 0 .. N-1-D+i
    pairs = 0
    for b in range(len(kv)):
        D = qs[b + 1] - qs[b] - 1
        for i in range(D + 1):
            for j in range(kv[b]):
                pairs += j <= kv[b] - 1 - D + i
    assert flops == pairs * sp.kv_heads * sp.group * sp.head_dim * 4
    T = int(qs[-1])
    kv_bytes = sum(int(n) * sp.kv_heads * sp.head_dim * 2 * 2 for n in kv)
    pages = sum((int(n) + 15) // 16 for n in kv)
    assert nbytes == kv_bytes + 2 * T * sp.kv_heads * sp.group * sp.head_dim * 2 + pages * 4


def test_accept_bytes():
    inp = generate(_spec())
    T, V = inp.target_logits.shape
    B = 3
    assert bench.algorithmic_accept(inp) == (T + (T - B)) * V * 4 + 2 * B * V * 4
    g = generate(_spec(mode="greedy"))
    assert bench.algorithmic_accept(g) == T * V * 4


def test_tree_flops_count_each_nodes_root_path():
    sp = _spec(batch=2, kv_len=[60, 33], draft_len=1)
    inp, parents, _ = tree_inputs(sp, (2, 2))
    nbytes, flops = bench.tree_algorithmic(inp, parents)
    par = parents.numpy()
    qs = inp.q_start.numpy()
    kv = inp.kv_len.numpy()
    pairs = 0
    for b in range(2):
        T = qs[b + 1] - qs[b] - 1
        p = par[qs[b] - b: qs[b] - b + T]
        for i in range(T + 1):
            depth, node = 0, i
            while node != 0:
                node = p[node - 1]
                depth += 1
            pairs += (kv[b] - 1 - T) + depth + 1
    assert flops == pairs * sp.kv_heads * sp.group * sp.head_dim * 4
    assert nbytes > sum(int(n) * sp.kv_heads * sp.head_dim * 4 for n in kv)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
