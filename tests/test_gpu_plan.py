"""GPU checks of the attention's device-side plan, through the C ABI: the
split-KV chunk it picks and the item and split-sequence counts it writes to the
head of the workspace, against the selection rule evaluated here directly (one
division per candidate chunk and sequence), on batches whose sequences are all
short, all long, mixed, or longer than the plan's LDS list of long sequences
holds; the work-item descriptors it writes (every (sequence, KV head, split)
exactly once, with its key range and fields, full-chunk items first, then the
shorter items longest first by length bucket, and the natural item index of
each sequence); and the attention output of the same calls against the oracle
on sampled (sequence, head) units.

The plan's chunk rule: candidates c(t), t < 256: 256 + 64 t keys for t < 240,
then 16384 + 1024 (t - 240) and 32768 for t = 255 (capped at the longest
sequence rounded up to 64, and at 32768); items(c) = H_kv * sum_b max(1,
ceil(N_b / c)); among the candidates whose items fit the workspace, the one
with the smallest max(ceil((H_kv * sum_b N_b + ovh * items(c)) / slots),
min(c, max_b N_b)) wins, the smaller c on ties; ovh = 192 KiB of K/V in keys,
slots = resident workgroups of the launch."""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_sd_amd as sdv
from tests.gpu_util import ATTN_TOL, compare_attention, on_gpu, say
from workloads import WorkloadSpec, generate

pytestmark = pytest.mark.gpu

PAGE = 16
MAX_CHUNK = 32768


def candidate(t):
    return 256 + 64 * t if t < 240 else 16384 + 1024 * (t - 240) if t < 255 else MAX_CHUNK


def expected_plan(kv, hkv, group, max_draft, head_dim, max_pages, cus, kv_chunk=0):
    """(chunk, items, sequences split in more than one item) by the rule above;
    the plan lists the split sequences only for batches whose combine would
    need more than 8192 workgroups of 8 rows (it writes 0 otherwise)."""
    n = np.minimum(np.maximum(np.asarray(kv, np.int64), 0), max_pages * PAGE)
    B = len(n)
    rmax = group * (1 + max_draft)
    per_cu = 2 if rmax <= 64 else 1
    slots = max(1, min(cus, 256) * per_cu)
    max_keys = max_pages * PAGE
    units = B * hkv
    if kv_chunk > 0:
        cap = units * -(-max_keys // kv_chunk)
    else:
        at_max = units * -(-max_keys // MAX_CHUNK)
        at_min = units * -(-max_keys // 256)
        cap = min(at_min, max(256 * per_cu * 4, at_max))
    cap = max(cap, 1)
    if kv_chunk > 0:
        chunk = kv_chunk
    else:
        cap_chunk = max(256, min(MAX_CHUNK, (max_keys + 63) // 64 * 64))
        ovh = 192 * 1024 // (4 * head_dim)
        best = None
        for t in range(256):
            c = min(candidate(t), cap_chunk)
            items = hkv * int(np.maximum(1, -(-n // c)).sum())
            if items > cap:
                continue
            load = (int(n.sum()) * hkv + ovh * items + slots - 1) // slots
            key = (max(load, min(c, int(n.max()))), t)
            best = key if best is None else min(best, key)
        chunk = cap_chunk if best is None else min(candidate(best[1]), cap_chunk)
    per_seq = np.maximum(1, -(-n // chunk))
    rpad = -(-rmax // 16) * 16
    listed = B * hkv * (rpad // 8) > 8192
    return chunk, hkv * int(per_seq.sum()), int((per_seq > 1).sum()) if listed else 0


def run_and_read_plan(inp, kv_chunk=0):
    x = on_gpu(inp)
    out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    desc = sdv.attn_desc(x.q, x.k_cache, x.block_table, inp.group, inp.max_draft, kv_chunk=kv_chunk)
    ws = torch.empty(sdv.sd_verify_attention_workspace_size(desc, x.q.shape[0]), dtype=torch.uint8, device="cuda")
    sdv.sd_verify_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start, out,
                            group_size=inp.group, max_draft=inp.max_draft, kv_chunk=kv_chunk, workspace=ws)
    torch.cuda.synchronize()
    # the plan header sits at the start of the workspace: chunk, items, full-chunk items, split sequences
    head = ws[:16].view(torch.int32).cpu().numpy()
    return out, int(head[0]), int(head[1]), int(head[3]), ws


def check_items(ws, inp, chunk, items):
    """The descriptors the plan wrote: 8 int32 each (b, h, k_begin, k_end, t0,
    D, N, nsplit) in schedule order after the plan header and its 4B+1 ints
    (item starts, shorter-item positions, split list, full-item bases), rounded
    up to 256 bytes; item_start[b] at int 16 + b."""
    B, hkv = inp.spec.batch, inp.spec.kv_heads
    off = -(-(16 + 4 * B + 1) * 4 // 256) * 256 // 4
    words = ws[:4 * (off + 8 * items)].view(torch.int32).cpu().numpy()
    desc = words[off:off + 8 * items].reshape(items, 8)
    kv = np.minimum(inp.kv_len.cpu().numpy().astype(np.int64), inp.block_table.shape[1] * PAGE)
    qs = inp.q_start.cpu().numpy()
    nsplit = np.maximum(1, -(-kv // chunk))
    seen = set()
    for b, h, k0, k1, t0, D, N, ns in desc.tolist():
        assert 0 <= b < B and 0 <= h < hkv
        assert (N, ns, t0, D) == (kv[b], nsplit[b], qs[b], qs[b + 1] - qs[b] - 1)
        assert k0 % chunk == 0 and k1 == min(N, k0 + chunk)
        seen.add((b, h, k0 // chunk))
    assert len(seen) == items == hkv * int(nsplit.sum())
    full = int(words[2])
    lens = desc[:, 3] - desc[:, 2]
    assert np.all(lens[:full] == chunk) and not np.any(lens[full:] == chunk)
    bucket = 63 - (lens[full:] * 64) // (chunk + 1)
    assert np.all(np.diff(bucket) >= 0), "shorter items longest first by bucket"
    start = np.concatenate([[0], np.cumsum(hkv * nsplit)[:-1]])
    assert np.array_equal(words[16:16 + B], start)


def spec(**kw):
    base = dict(name="plan_case", batch=4, kv_heads=2, group=4, head_dim=64, kv_len=100, draft_len=3,
                vocab=64, mode="greedy")
    base.update(kw)
    return WorkloadSpec(**base)


def check(inp, kv_chunk=0, units=None):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sp = inp.spec
    want = expected_plan(inp.kv_len.cpu().numpy(), sp.kv_heads, sp.group, inp.max_draft, sp.head_dim,
                         inp.block_table.shape[1], cus, kv_chunk)
    out, chunk, items, nsplit, ws = run_and_read_plan(inp, kv_chunk)
    say(f"  plan: chunk {chunk}, items {items}, split sequences {nsplit} (expected {want})")
    assert (chunk, items, nsplit) == want
    check_items(ws, inp, chunk, items)
    err = compare_attention(inp, out, units=units)
    say(f"  max|err| over {len(units) if units else 'all'} units = {err:.3e}")
    assert err <= ATTN_TOL


def test_all_short_sequences_large_batch():
    """4096 sequences of 200 keys: no split, the combine visits nothing."""
    inp = generate(spec(batch=4096, kv_heads=1, group=2, kv_len=200, draft_len=1, seed=31))
    say("case: plan B=4096 N=200")
    check(inp, units=[(0, 0), (1234, 0), (4095, 0)])


def test_all_long_sequences():
    """16 sequences of 32768 keys over 2 heads (the plan's longest histogram
    bin), split in several items to fill the GPU."""
    inp = generate(spec(batch=16, kv_heads=2, group=8, kv_len=32768, draft_len=7, seed=32))
    say("case: plan B=16 N=32768")
    check(inp, units=[(0, 0), (7, 1), (15, 1)])


def test_mixed_lengths_with_some_long():
    rng = np.random.default_rng(33)
    kv = [int(x) for x in rng.integers(1, 1500, size=2500)]
    for b in (3, 700, 2100):
        kv[b] = int(rng.integers(33000, 60000))
    inp = generate(spec(batch=2500, kv_heads=1, group=2, kv_len=kv, draft_len=[int(x) for x in rng.integers(0, 4, size=2500)],
                        seed=33))
    say("case: plan B=2500 mixed, 3 long")
    check(inp, units=[(3, 0), (700, 0), (2100, 0), (5, 0), (2499, 0)])


def test_more_long_sequences_than_the_plan_lists():
    """260 sequences just over 32768 keys: more than the 256 the chunk search
    lists in LDS, so it counts every sequence directly."""
    inp = generate(spec(batch=260, kv_heads=1, group=1, kv_len=32800, draft_len=0, seed=34))
    say("case: plan B=260 N=32800")
    check(inp, units=[(0, 0), (259, 0)])


def test_large_batch_every_sequence_split():
    """1100 sequences over 8 row blocks each (8800 combine workgroups), all
    split by a 512-key chunk: the combine walks the plan's list of split
    sequences."""
    rng = np.random.default_rng(36)
    kv = [int(x) for x in rng.integers(600, 2000, size=1100)]
    inp = generate(spec(batch=1100, kv_heads=1, group=8, kv_len=kv, draft_len=7, seed=36))
    say("case: plan B=1100 kv_chunk=512, listed splits")
    check(inp, kv_chunk=512, units=[(0, 0), (549, 0), (1099, 0)])


def test_explicit_chunk_counts_split_sequences():
    inp = generate(spec(batch=6, kv_len=[100, 256, 257, 1000, 5, 513], seed=35))
    say("case: plan kv_chunk=256")
    check(inp, kv_chunk=256)


@pytest.mark.parametrize("batch", [32, 33])
def test_mixed_lengths_at_the_fused_limit(batch):
    """Uneven lengths with shorter items in several length buckets: 32
    sequences plan inside the main kernel (fixed-stride schedule), 33 take the
    plan kernel (dynamic schedule); both by the same selection rule."""
    rng = np.random.default_rng(40 + batch)
    kv = [int(x) for x in rng.integers(1, 9000, size=batch)]
    inp = generate(spec(batch=batch, kv_heads=2, group=8, kv_len=kv,
                        draft_len=[int(x) for x in rng.integers(0, 8, size=batch)], seed=40 + batch))
    say(f"case: plan B={batch} mixed lengths")
    check(inp, units=[(0, 0), (batch // 2, 1), (batch - 1, 1)])


def test_fused_plan_with_listed_splits():
    """32 sequences over 32 KV heads at 128 rows each (16384 combine workgroups
    of 8 rows): the plan made inside the main kernel also writes the list of
    split sequences the combine walks."""
    rng = np.random.default_rng(42)
    kv = [int(x) for x in rng.integers(300, 3000, size=32)]
    inp = generate(spec(batch=32, kv_heads=32, group=8, kv_len=kv, draft_len=15, seed=42))
    say("case: plan B=32 Hkv=32, listed splits")
    check(inp, kv_chunk=512, units=[(0, 0), (13, 31), (31, 7)])
