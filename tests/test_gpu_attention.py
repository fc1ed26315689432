"""GPU parity of verify attention against the fp64 oracle (|err| <= 2e-2 on
bf16 outputs), through the C ABI.  Sizes span several 64-key tiles, ragged
page tails, split-KV with the combine pass, every row-block variant
(G*(1+D) up to 64, 128 and 256) and both head dims."""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_sd_amd as sdv

from tests.gpu_util import ATTN_TOL, compare_attention, gpu_attention, on_gpu, say
from workloads import WorkloadSpec, generate, preset

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="attn_case", batch=3, kv_heads=2, group=8, head_dim=128, kv_len=[1000, 77, 2500],
                draft_len=[15, 3, 7], vocab=64, mode="stochastic")
    base.update(kw)
    return WorkloadSpec(**base)


def test_tiny_workload_full_parity():
    inp = generate(preset("tiny"))
    say("case: tiny d=64")
    err = compare_attention(inp, gpu_attention(inp))
    say(f"tiny max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("kv_chunk", [0, 256, 64, 8192])
def test_ragged_lengths_and_split_kv(kv_chunk):
    inp = generate(spec())
    say(f"case: ragged G=8 d=128 kv_chunk={kv_chunk}")
    err = compare_attention(inp, gpu_attention(inp, kv_chunk=kv_chunk))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("G,drafts,d", [
    (8, [0, 0], 128),          # R = 8 (plain decode)
    (4, [3, 2], 64),           # R = 16
    (8, [3, 1], 128),          # R <= 64
    (8, [15, 9], 128),         # R <= 128
    (8, [31, 20], 128),        # R <= 256
    (8, [16, 9], 128),         # R = 136: rows 128..143 a 16-row block, split by tile parity
    (16, [8, 3], 128),         # R = 144: the 16-row block full
    (5, [27, 3], 128),         # R = 140
    (4, [35, 20], 64),         # R = 144, d = 64
    (8, [23, 19], 128),        # R = 192
    (12, [15, 10], 64),        # R = 192, d = 64
    (3, [50, 47], 128),        # R = 153
    (32, [3, 1], 128),         # G = 32, R = 128
    (32, [7, 2], 128),         # G = 32, R = 256
    (16, [15, 4], 64),         # R = 256, d = 64
    (1, [0, 7], 128),          # G = 1
])
def test_row_block_variants(G, drafts, d):
    inp = generate(spec(batch=2, group=G, head_dim=d, kv_len=[700, 1333], draft_len=drafts, seed=G + d))
    say(f"case: G={G} drafts={drafts} d={d}")
    err = compare_attention(inp, gpu_attention(inp, kv_chunk=256))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL
    err = compare_attention(inp, gpu_attention(inp))
    assert err <= ATTN_TOL


def test_maximum_fixed_chunk_splits():
    """kv_chunk at its maximum (8192 keys) on caches of 20000 and 8193 keys:
    three and two splits merged by the combine, and a short cache unsplit."""
    inp = generate(spec(kv_len=[20000, 8193, 300], seed=11))
    say("case: kv_chunk=8192 with splits")
    err = compare_attention(inp, gpu_attention(inp, kv_chunk=8192))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


def _dim_major(inp):
    """The same inputs with each V page stored d-major ([P, H, d, page])."""
    x = on_gpu(inp)
    dm = x.v_cache.transpose(2, 3).contiguous()
    return x, dm


@pytest.mark.parametrize("G,drafts,d,kv_chunk", [
    (8, [0, 0], 128, 0),         # R = 8
    (4, [3, 2], 64, 256),        # R = 16, d = 64, split
    (8, [7, 5], 128, 0),         # R = 64
    (8, [15, 9], 128, 256),      # R = 128 (the wave sets split the tiles)
    (8, [16, 9], 128, 0),        # R = 136 (rows past 128: a 16-row block split by tile parity)
    (8, [16, 9], 128, 256),      # R = 136, split
    (4, [35, 20], 64, 0),        # R = 144, d = 64
    (8, [31, 20], 128, 256),     # R = 256 (row split)
    (16, [15, 4], 64, 0),        # R = 256, d = 64
])
def test_dim_major_v_cache(G, drafts, d, kv_chunk):
    """V pages stored d-major ([P, H_kv, d, 16]): the kernels copy the V^T
    operand straight from the page and must give exactly the output of the
    key-major call (transposing LDS loads; the same bf16 operands in the same
    order), which matches the oracle; the page tails past each sequence are NaN."""
    inp = generate(spec(batch=2, group=G, head_dim=d, kv_len=[1700, 1333], draft_len=drafts, seed=3 * G + d),
                   poison_tail=True)
    x, dm = _dim_major(inp)
    say(f"case: d-major V G={G} drafts={drafts} d={d} kv_chunk={kv_chunk}")
    ref = gpu_attention(inp, kv_chunk=kv_chunk)
    out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    sdv.sd_verify_attention(x.q, x.k_cache, dm, x.block_table, x.kv_len, x.q_start, out, group_size=inp.group,
                            max_draft=inp.max_draft, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    err = compare_attention(inp, out)
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


def test_dim_major_v_cache_full_size():
    """The benchmarked default shape with a d-major V cache: bit-identical to
    the key-major call and equal to the oracle on every element."""
    sp = preset("g8_kv32k_D15")
    inp = generate(sp, device="cuda")
    say(f"case: full size {sp.name}, d-major V")
    ref = gpu_attention(inp)
    dm = inp.v_cache.transpose(2, 3).contiguous()
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    sdv.sd_verify_attention(inp.q, inp.k_cache, dm, inp.block_table, inp.kv_len, inp.q_start, out,
                            group_size=inp.group, max_draft=inp.max_draft)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    err = compare_attention(inp, out)
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("drafts", [[16, 12, 2], [23, 19, 17], [31, 25, 0]])
def test_long_items_every_row_block(drafts):
    """Items of thousands of keys (the unrolled steady loop runs many groups) at
    136, 192 and 256 rows per KV head: every 32-row block, whichever wave and
    tile parity serves it, matches the oracle."""
    inp = generate(spec(batch=3, group=8, kv_len=[9000, 5000, 7001], draft_len=drafts, seed=sum(drafts)))
    say(f"case: long items drafts={drafts}")
    err = compare_attention(inp, gpu_attention(inp))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("kv_chunk", [0, 256])
def test_many_sequences_mixed_lengths(kv_chunk):
    """More sequences than the plan keeps in LDS (8192), lengths 1..300 plus one
    long sequence: the plan's global path, items shorter than the chunk in
    longest-first order, and workgroups taking items from the counters.
    Checked on sampled units, the long one, and sequences on both sides of
    the LDS boundary."""
    rng = np.random.default_rng(21)
    B = 8300
    kv = [int(x) for x in rng.integers(1, 300, size=B)]
    kv[0] = 20000
    dr = [int(x) for x in rng.integers(0, 4, size=B)]
    inp = generate(spec(batch=B, kv_heads=1, group=2, head_dim=64, kv_len=kv, draft_len=dr, seed=21))
    say(f"case: B={B} mixed lengths kv_chunk={kv_chunk}")
    units = [(0, 0)] + [(int(b), 0) for b in rng.choice(B, size=60, replace=False)] + \
        [(b, 0) for b in (8190, 8191, 8192, 8193, B - 1)]
    err = compare_attention(inp, gpu_attention(inp, kv_chunk=kv_chunk), units=units)
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("drafts", [[15, 3, 7], [16, 3, 7]])
def test_fp32_output_and_explicit_scale(drafts):
    inp = generate(spec(seed=4, draft_len=drafts))
    say(f"case: fp32 output, scale 0.05, drafts {drafts}")
    from oracle import verify_attention
    from tests.oracle_io import attention_args
    ref = verify_attention(**attention_args(inp), scale=0.05)
    out = gpu_attention(inp, out_dtype=torch.float32, softmax_scale=0.05).cpu().numpy()
    err = float(np.abs(out - ref).max())
    say(f"max|err| = {err:.3e}")
    assert err <= 1e-2


def test_nan_past_the_sequence_end_is_never_read():
    inp = generate(spec(kv_len=[1001, 77, 35], seed=5), poison_tail=True)
    say("case: NaN-poisoned page tails")
    for chunk in (0, 64):
        err = compare_attention(inp, gpu_attention(inp, kv_chunk=chunk))
        assert err <= ATTN_TOL


def test_sequence_shorter_than_its_block():
    inp = generate(spec(batch=2, kv_len=[3, 16], draft_len=[5, 15], seed=6))
    say("case: kv_len < 1+D")
    out = gpu_attention(inp)
    err = compare_attention(inp, out)
    assert err <= ATTN_TOL
    assert torch.all(out[0:3].float() == 0)


def test_deterministic():
    inp = generate(spec(seed=7))
    a = gpu_attention(inp, kv_chunk=256)
    b = gpu_attention(inp, kv_chunk=256)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("G,drafts,kv,kv_chunk", [
    (8, [0, 0], [700, 1333], 0),                  # plain decode, split-KV with the combine
    (8, [15, 9], [700, 1333], 0),                 # R <= 128
    (8, [31, 20], [700, 1333], 0),                # R <= 256 (row split)
    (8, [19, 12], [700, 1333], 0),                # R = 160 (blocks 4-5 split by tile parity)
    (8, [16, 12], [700, 1333], 0),                # R = 136 (a 16-row block split by tile parity)
    (2, [3, 0, 1, 2] * 40, [37, 900, 5000, 260] * 40, 0),   # short items: counter-driven fetch
    # caches of at most 256 keys: never split, and no combine launch (plan in the
    # main kernel for B <= 32, the plan kernel past that)
    (8, [3, 7, 0, 15], [256, 9, 200, 17], 0),
    (4, [3, 1, 0, 2] * 12, [256, 129, 64, 250] * 12, 0),
])
def test_workspace_contents_never_matter(G, drafts, kv, kv_chunk):
    """The call initialises every workspace byte it reads: with the workspace
    filled with different byte patterns before each call, every call returns
    the same bits, and they match the oracle."""
    inp = generate(spec(batch=len(kv), group=G, kv_len=kv, draft_len=drafts, seed=31))
    x = inp.to("cuda")
    desc = sdv.attn_desc(x.q, x.k_cache, x.block_table, inp.group, inp.max_draft, kv_chunk=kv_chunk)
    nbytes = sdv.sd_verify_attention_workspace_size(desc, x.q.shape[0])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    outs = []
    for rep, fill in enumerate([0xFF, 0x00, 0x7F, 0x80, None, 0xFF, None, 0x00]):
        if fill is None:
            ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen))
        else:
            ws.fill_(fill)
        out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        sdv.sd_verify_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start, out,
                                group_size=inp.group, max_draft=inp.max_draft, kv_chunk=kv_chunk, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    say(f"case: workspace garbage G={G} B={len(kv)}")
    for rep, o in enumerate(outs[1:], 1):
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), f"call {rep} differs from call 0"
    err = compare_attention(inp, outs[0])
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("name,over", [
    ("g8_kv32k_D15", {}),                          # B16 G8 32K keys, D=15 (128 rows per KV head)
    ("g32_kv128k_D3_greedy", {}),                  # B4 G32 128K keys, D=3 (128 rows)
    ("g8_kv32k_sweep", dict(draft_len=0)),         # B32 G8 32K keys: 8 rows (plain decode)
    ("g8_kv32k_sweep", dict(draft_len=15)),        # 128 rows
    ("g8_kv32k_sweep", dict(draft_len=16)),        # 136 rows
    ("g8_kv32k_sweep", dict(draft_len=23)),        # 192 rows
    ("g8_kv32k_sweep", dict(draft_len=31)),        # 256 rows
    ("ragged_b64", {}),                            # B64 lognormal 1K..128K keys, D in {3, 7, 15}
])
def test_full_size_full_output(name, over):
    """The benchmarked shapes in the launch configuration bench.py times: every
    output element is compared with the oracle (run on the host threads), and
    no element of the NaN-prefilled output may be left unwritten."""
    sp = preset(name, **over)
    say(f"case: full size {sp.name}")
    inp = generate(sp, device="cuda")
    out = gpu_attention(inp)
    assert not torch.isnan(out.float()).any(), "unwritten output rows"
    err = compare_attention(inp, out)
    say(f"{sp.name}: max|err| over every element = {err:.3e}")
    assert err <= ATTN_TOL


def _plant_dominant_key(inp, b, h, key, scale=5.0, negative_prefix=0):
    """All queries of KV head h get one vector v; key `key` of sequence b becomes
    scale*v (a score far above anything before it), optionally after a prefix of
    keys pointing away from v (scores far below)."""
    G = inp.group
    g = torch.Generator().manual_seed(1234 + key)
    v = torch.randn(inp.q.shape[-1], generator=g).to(torch.bfloat16)
    inp.q[:, h * G:(h + 1) * G, :] = v
    bt = inp.block_table[b].cpu()
    ps = inp.spec.page_size
    inp.k_cache[int(bt[key // ps]), h, key % ps, :] = (scale * v.float()).to(torch.bfloat16)
    for j in range(negative_prefix):
        inp.k_cache[int(bt[j // ps]), h, j % ps, :] = (-scale * v.float()).to(torch.bfloat16)


@pytest.mark.parametrize("key,prefix,kv_chunk,D", [
    (2000, 0, 0, 7),       # late dominant key, one item per sequence
    (2000, 0, 256, 7),     # ... in a later split
    (2497, 0, 0, 7),       # inside the draft block (visible to the last rows only)
    (1500, 32, 0, 7),      # first tile far below everything after it
    (2000, 0, 256, 16),    # 136 rows: the 16-row block's safe pass too
    (2497, 0, 0, 16),
    (1500, 32, 0, 16),
])
def test_score_far_above_the_first_tile_max(key, prefix, kv_chunk, D):
    inp = generate(spec(batch=1, kv_len=[2500], draft_len=[D], seed=5))
    _plant_dominant_key(inp, 0, 1, key, negative_prefix=prefix)
    say(f"case: dominant key {key} prefix {prefix} kv_chunk={kv_chunk} D={D}")
    err = compare_attention(inp, gpu_attention(inp, kv_chunk=kv_chunk))
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("group,kv_chunk,D", [(8, 0, 7), (8, 512, 7), (16, 512, 7), (8, 512, 16)])
def test_dynamic_schedule_many_items_per_workgroup(group, kv_chunk, D):
    """1100 sequences of 600..2000 keys with D=7 (64 rows per KV head: every wave
    of the R <= 64 kernel has rows; group 16: the wide kernel) or D=16 (136
    rows: the 16-row block, whose safe-pass votes go through LDS slots reused
    item after item), several items per workgroup handed out by the work
    counters.  Each wave must take the
    item index the counter gave its workgroup: the index passes through LDS,
    and a barrier does not wait for LDS stores by itself (a wave that read the
    old index redid the previous item and left its rows of the new one
    unwritten).  Three workspace fills give bit-identical outputs with every
    row written, and sampled units (late, dynamically scheduled items
    included) match the oracle."""
    rng = np.random.default_rng(37)
    B = 1100
    kv = [int(x) for x in rng.integers(600, 2000, size=B)]
    inp = generate(spec(batch=B, kv_heads=1, group=group, head_dim=64, kv_len=kv, draft_len=D, seed=37))
    x = on_gpu(inp)
    desc = sdv.attn_desc(x.q, x.k_cache, x.block_table, group, inp.max_draft, kv_chunk=kv_chunk)
    n = sdv.sd_verify_attention_workspace_size(desc, x.q.shape[0])
    say(f"case: dynamic schedule B={B} G={group} D={D} kv_chunk={kv_chunk}")
    outs = []
    for fill in ("zeros", "ones", "random"):
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(255)
        else:
            ws.copy_(torch.randint(0, 256, (n,), dtype=torch.uint8))
        out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        sdv.sd_verify_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start, out,
                                group_size=group, max_draft=inp.max_draft, kv_chunk=kv_chunk, workspace=ws)
        torch.cuda.synchronize()
        assert not torch.isnan(out.float()).any(), f"unwritten rows with a {fill} workspace"
        outs.append(out.cpu())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    units = [(int(b), 0) for b in rng.choice(B, size=24, replace=False)] + [(B - 1, 0), (B - 2, 0)]
    err = compare_attention(inp, outs[0], units=units)
    say(f"max|err| = {err:.3e}")
    assert err <= ATTN_TOL
