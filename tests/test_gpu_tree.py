"""GPU parity of draft-tree verification against the fp64 tree oracle, through
the C ABI: attention under the ancestor mask (|err| <= 2e-2 on bf16 outputs;
a chain tree must give the causal call's output bit for bit) and greedy
acceptance of the longest accepted path (bit-exact lengths, tokens and nodes)."""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_sd_amd as sdv
from oracle import accept_tree_greedy, verify_tree_attention
from tests.gpu_util import ATTN_TOL, gpu_attention, say
from tests.oracle_io import attention_args
from workloads import WorkloadSpec, generate

pytestmark = pytest.mark.gpu


def _spec(**kw):
    base = dict(name="tree_case", batch=3, kv_heads=2, group=8, head_dim=128, kv_len=[1000, 77, 2500],
                draft_len=[15, 3, 7], vocab=64, mode="greedy")
    base.update(kw)
    return WorkloadSpec(**base)


def _parents(q_start, kind, rng):
    par = []
    for b in range(len(q_start) - 1):
        T = int(q_start[b + 1] - q_start[b]) - 1
        for i in range(1, T + 1):
            par.append(i - 1 if kind == "chain" else 0 if kind == "star" else int(rng.integers(0, i)))
    return np.asarray(par, np.int32)


def _tree_attention(inp, parents, kv_chunk=0):
    x = inp if inp.q.is_cuda else inp.to("cuda")
    out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    sdv.sd_verify_tree_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start,
                                 torch.from_numpy(parents).cuda(), out, group_size=inp.group,
                                 max_draft=inp.max_draft, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("G,drafts,d", [(8, [3, 1, 7], 128), (8, [15, 9, 4], 128), (8, [31, 20, 5], 128),
                                        (4, [63, 30, 0], 64), (8, [16, 9, 4], 128)])
def test_chain_tree_is_bitwise_the_causal_call(G, drafts, d):
    inp = generate(_spec(group=G, head_dim=d, draft_len=drafts, seed=G + d))
    par = _parents(inp.q_start.cpu().numpy(), "chain", None)
    say(f"case: chain G={G} drafts={drafts} d={d}")
    a = _tree_attention(inp, par)
    c = gpu_attention(inp)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("kind", ["random", "star"])
@pytest.mark.parametrize("G,drafts,d,kv_chunk", [(8, [15, 3, 7], 128, 0), (8, [31, 12, 6], 128, 0),
                                                 (4, [7, 2, 5], 64, 0), (8, [15, 3, 7], 128, 256),
                                                 (2, [40, 63, 1], 64, 0), (3, [50, 20, 7], 128, 0),
                                                 (3, [50, 20, 7], 128, 256), (8, [16, 3, 7], 128, 0),
                                                 (8, [16, 3, 7], 128, 256), (4, [35, 20, 1], 64, 0)])
def test_tree_attention_matches_oracle(kind, G, drafts, d, kv_chunk):
    inp = generate(_spec(group=G, head_dim=d, draft_len=drafts, seed=3 * G + d + len(kind)))
    rng = np.random.default_rng(G + d)
    a = attention_args(inp)
    par = _parents(a["q_start"], kind, rng)
    say(f"case: {kind} tree G={G} drafts={drafts} d={d} kv_chunk={kv_chunk}")
    out = _tree_attention(inp, par, kv_chunk).float().cpu().numpy().astype(np.float64)
    ref = verify_tree_attention(parents=par, **a)
    err = float(np.max(np.abs(out - ref)))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("kind", ["random", "star"])
@pytest.mark.parametrize("G,kv_chunk", [(1, 64), (1, 128), (2, 64), (3, 64), (4, 64), (4, 128)])
def test_split_boundary_inside_the_tree(kind, G, kv_chunk):
    """64-node trees whose last split begins inside the tree (1, 10 and 30 nodes
    in), with G = 1 (64 rows: the R <= 64 kernel), G = 2 (128 rows: the wide
    kernel whose wave sets split the tiles), G = 3 (192 rows: rows past 128
    split by tile parity) and G = 4 (256 rows: the row-split wide kernel).  A node whose root path has no node in the first
    tile of that split sees no key there, yet sees its own nodes in a later
    tile of the split: its partial must still enter the combine with the
    offset its values were computed against."""
    kv = [1087, 1078, 1058]                   # tree starts at key 1023, 1014 and 994; a split starts at 1024
    inp = generate(_spec(batch=3, group=G, head_dim=128, kv_len=kv, draft_len=[63, 63, 63], seed=40 + G))
    rng = np.random.default_rng(41 + G)
    a = attention_args(inp)
    par = _parents(a["q_start"], kind, rng)
    say(f"case: split inside the tree, {kind} tree G={G} kv_chunk={kv_chunk}")
    out = _tree_attention(inp, par, kv_chunk)
    assert not torch.isnan(out.float()).any()
    ref = verify_tree_attention(parents=par, **a)
    err = float(np.max(np.abs(out.float().cpu().numpy().astype(np.float64) - ref)))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("kind", ["random", "star"])
@pytest.mark.parametrize("kv_chunk", [64, 128])
def test_split_boundary_inside_the_tree_16_row_block(kind, kv_chunk):
    """36-node trees at G = 4 (144 rows: the rows past 128 are one 16-row
    block) whose last split begins 1, 10 and 30 nodes into the tree: as above,
    with the 16-row block's own reference max and partial."""
    kv = [1059, 1050, 1030]                   # tree starts at key 1023, 1014 and 994; a split starts at 1024
    inp = generate(_spec(batch=3, group=4, head_dim=128, kv_len=kv, draft_len=[35, 35, 35], seed=60))
    rng = np.random.default_rng(61)
    a = attention_args(inp)
    par = _parents(a["q_start"], kind, rng)
    say(f"case: split inside the tree, 16-row block, {kind} tree kv_chunk={kv_chunk}")
    out = _tree_attention(inp, par, kv_chunk)
    assert not torch.isnan(out.float()).any()
    ref = verify_tree_attention(parents=par, **a)
    err = float(np.max(np.abs(out.float().cpu().numpy().astype(np.float64) - ref)))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("G,drafts,kv_chunk", [(1, [63, 40, 2], 64), (8, [15, 9, 4], 0), (4, [63, 31, 1], 128),
                                               (4, [35, 31, 1], 128)])
def test_tree_dim_major_v_cache(G, drafts, kv_chunk):
    """Tree attention over a d-major V cache equals the key-major call bit for bit."""
    inp = generate(_spec(group=G, draft_len=drafts, kv_len=[1087, 900, 2500], seed=50 + G))
    par = _parents(attention_args(inp)["q_start"], "random", np.random.default_rng(51))
    x = inp.to("cuda")
    dm = x.v_cache.transpose(2, 3).contiguous()
    say(f"case: tree d-major V G={G} drafts={drafts} kv_chunk={kv_chunk}")
    ref = _tree_attention(x, par, kv_chunk)
    out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    sdv.sd_verify_tree_attention(x.q, x.k_cache, dm, x.block_table, x.kv_len, x.q_start,
                                 torch.from_numpy(par).cuda(), out, group_size=inp.group, max_draft=inp.max_draft,
                                 kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("G,drafts", [(8, [3, 1, 7]), (8, [15, 9, 4]), (8, [31, 20, 5])])
def test_tree_workspace_contents_never_matter(G, drafts):
    """The tree masks and the plan are written by the call before they are
    read: different workspace fills give the same bits every call."""
    inp = generate(_spec(group=G, draft_len=drafts, seed=G + 1))
    par = _parents(attention_args(inp)["q_start"], "random", np.random.default_rng(7))
    x = inp.to("cuda")
    desc = sdv.attn_desc(x.q, x.k_cache, x.block_table, inp.group, inp.max_draft)
    nbytes = sdv.sd_verify_attention_workspace_size(desc, x.q.shape[0])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    parents = torch.from_numpy(par).cuda()
    say(f"case: tree workspace garbage G={G} drafts={drafts}")
    outs = []
    for fill in (0xFF, 0x00, 0x7F, 0x80, 0x55):
        ws.fill_(fill)
        out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        sdv.sd_verify_tree_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start, parents, out,
                                     group_size=inp.group, max_draft=inp.max_draft, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    ref = verify_tree_attention(parents=par, **attention_args(inp))
    err = float(np.max(np.abs(outs[0].float().cpu().numpy() - ref)))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


def _run_accept(target, tokens, q_start, parents, max_draft):
    T = target.shape[0]
    B = q_start.shape[0] - 1
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    nodes = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    sdv.sd_tree_accept(target, tokens, q_start, parents, al, out, nodes, max_draft=max_draft)
    torch.cuda.synchronize()
    return al.cpu().numpy(), out.cpu().numpy(), nodes.cpu().numpy()


@pytest.mark.parametrize("seed,V", [(0, 5), (1, 7), (2, 1001), (3, 32000), (4, 151936)])
def test_tree_accept_matches_oracle(seed, V):
    rng = np.random.default_rng(seed)
    B = 6
    sizes = rng.integers(1, 30, size=B)
    sizes[0] = 1                              # a sequence with no drafts
    q_start = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(q_start[-1])
    target = rng.standard_normal((T, V)).astype(np.float32) * 3
    parents = _parents(q_start, "random", rng)
    tokens = rng.integers(0, V, size=T - B).astype(np.int32)
    for b in range(B):                        # plant matches so that paths get long
        t0, d0 = int(q_start[b]), int(q_start[b]) - b
        for i in range(1, int(sizes[b])):
            if rng.random() < 0.7:
                tokens[d0 + i - 1] = int(np.argmax(target[t0 + parents[d0 + i - 1]]))
    tokens[rng.random(T - B) < 0.05] = -3     # out-of-range drafts fail
    say(f"case: tree accept seed={seed} V={V}")
    got = _run_accept(torch.from_numpy(target).cuda(), torch.from_numpy(tokens).cuda(),
                      torch.from_numpy(q_start).cuda(), torch.from_numpy(parents).cuda(), int(sizes.max()) - 1)
    ref = accept_tree_greedy(target, tokens, q_start, parents)
    for g, r, name in zip(got, ref, ("accept_len", "out_tokens", "out_nodes")):
        np.testing.assert_array_equal(g, r, err_msg=name)
    say(f"AL = {got[0].tolist()}")


def test_full_size_tree_workload():
    """The benchmarked tree-verify step (16 sequences, G = 8, 32768-token caches,
    a full binary tree of depth 4, 131072-token vocabulary) in the launch
    configuration bench.py times: every attention output element against the
    tree oracle (run on the host threads), and the whole greedy tree
    acceptance bit-exact."""
    from tests.gpu_util import oracle_workers
    from workloads import preset
    from workloads.tree import tree_inputs
    sp = preset("g8_kv32k_D15")
    inp, parents, tokens = tree_inputs(sp, (2, 2, 2, 2), device="cuda")
    say("case: full-size tree verify step")
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    sdv.sd_verify_tree_attention(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start,
                                 parents, out, group_size=sp.group, max_draft=inp.max_draft)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any(), "unwritten output rows"
    par = parents.cpu().numpy()
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            ref = verify_tree_attention(parents=par, workers=oracle_workers(), **attention_args(inp))
    except ImportError:
        ref = verify_tree_attention(parents=par, workers=oracle_workers(), **attention_args(inp))
    worst = float(np.max(np.abs(out.float().cpu().numpy().astype(np.float64) - ref)))
    say(f"tree attention max|err| over every element = {worst:.3e}")
    assert worst <= ATTN_TOL
    got = _run_accept(inp.target_logits, tokens, inp.q_start, parents, inp.max_draft)
    ref = accept_tree_greedy(inp.target_logits.cpu().numpy(), tokens.cpu().numpy(), inp.q_start.cpu().numpy(), par)
    for g, r, name in zip(got, ref, ("accept_len", "out_tokens", "out_nodes")):
        np.testing.assert_array_equal(g, r, err_msg=name)
    say(f"mean AL = {got[0].mean():.3f}")


@pytest.mark.parametrize("group", [8, 16])
def test_tree_dynamic_schedule_many_items_per_workgroup(group):
    """900 sequences of 600..2000 keys with random trees of 7 nodes (64 or 128
    rows per KV head: the R <= 64 kernel and the wide kernel, tree variants)
    and a 512-key chunk, so that workgroups take several items each from the
    work counters (whose index reaches the waves through LDS).  Three
    workspace fills give bit-identical outputs with every row written;
    sampled units match the tree oracle."""
    rng = np.random.default_rng(38)
    B = 900
    kv = [int(x) for x in rng.integers(600, 2000, size=B)]
    inp = generate(_spec(batch=B, kv_heads=1, group=group, head_dim=64, kv_len=kv, draft_len=7, seed=38))
    args = attention_args(inp)
    par = _parents(args["q_start"], "random", rng)
    x = inp.to("cuda")
    parents = torch.from_numpy(par).cuda()
    desc = sdv.attn_desc(x.q, x.k_cache, x.block_table, inp.group, inp.max_draft, kv_chunk=512)
    nbytes = sdv.sd_verify_attention_workspace_size(desc, x.q.shape[0])
    say(f"case: tree dynamic schedule B={B} G={group}")
    outs = []
    for fill in (0x00, 0xFF, 0x5A):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        sdv.sd_verify_tree_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start, parents, out,
                                     group_size=inp.group, max_draft=inp.max_draft, kv_chunk=512, workspace=ws)
        torch.cuda.synchronize()
        assert not torch.isnan(out.float()).any(), f"unwritten rows with workspace fill {fill:#x}"
        outs.append(out.cpu())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    units = [(int(b), 0) for b in rng.choice(B, size=16, replace=False)] + [(B - 1, 0)]
    ref = verify_tree_attention(parents=par, units=units, **args)
    got = outs[0].float().numpy().astype(np.float64)
    mask = ~np.isnan(ref)
    err = float(np.max(np.abs(got[mask] - ref[mask])))
    say(f"max|err| over {len(units)} units = {err:.3e}")
    assert err <= ATTN_TOL
