"""Benchmark of one speculative-decoding verify step on one MI355X.

A step is one verify-attention call plus one accept/reject call over one batch
of seeded synthetic inputs already resident in HBM (the two halves of
sd_verify_step, timed separately with HIP events on the stream they run on).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--draft D] [--alpha A]
                    [--no-cpu-baseline] [--json-only]

Prints one JSON line.  The default workload is 16 sequences x 8 KV heads x
G=8 over a 32768-token paged bf16 cache with D=15 drafts (G*(1+D) = 128) and
stochastic acceptance over a 131072-token vocabulary.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified tokens/s per verify step (B,G,D,KV sweep) + % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def algorithmic_attention(inp):
    """Bytes and flops one attention call must move / do (masked keys and padding excluded)."""
    import numpy as np
    kv = inp.kv_len.cpu().numpy().astype(np.int64)
    qs = inp.q_start.cpu().numpy().astype(np.int64)
    D = np.diff(qs) - 1
    sp = inp.spec
    d, Hkv, G = sp.head_dim, sp.kv_heads, sp.group
    T = int(qs[-1])
    kv_bytes = int((kv * Hkv * d * 2 * 2).sum())
    q_bytes = T * Hkv * G * d * 2
    o_bytes = q_bytes
    bt_bytes = int(((kv + sp.page_size - 1) // sp.page_size).sum()) * 4
    visible = 0
    for b in range(len(kv)):
        i = np.arange(D[b] + 1)
        visible += int(np.maximum(kv[b] - D[b] + i, 0).sum())
    flops = 4 * d * Hkv * G * visible
    return kv_bytes + q_bytes + o_bytes + bt_bytes, flops


def algorithmic_accept(inp):
    sp = inp.spec
    T = inp.target_logits.shape[0]
    B = inp.q_start.shape[0] - 1
    V = sp.vocab
    if sp.mode == "greedy":
        return T * V * 4
    return (2 * T - B) * V * 4 + 2 * B * V * 4   # one pass over all rows + the residual/bonus rows


def cpu_info():
    """Host CPUs the oracle may use here, the host's total and its model name."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):        # pragma: no cover
        usable = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:                           # pragma: no cover
        pass
    return usable, os.cpu_count() or usable, model


# The GPU machine gives one GPU a share of 16 host cores, whatever the host's total:
# the oracle's pool is sized to that share (or fewer, where fewer are usable).
ORACLE_THREADS = 16


def cpu_baseline(inp, budget_s: float = 20.0, gpu_out=None, gpu_al=None, gpu_tok=None, tol: float = 2e-2):
    """Time the oracle on the host cores over the same workload, and compare its
    results with the GPU's outputs of the same inputs.

    Attention units (sequence, KV head) are taken in a seeded random order and
    run in batches on a thread pool until every unit is done or `budget_s` has
    passed; then the same for the sequences' accept/reject.  The measured time
    is scaled by units done / units in the step (1.0 when the whole step ran).
    With the GPU's outputs given, every unit the oracle ran is compared with
    them: attention element by element (max |err| and the count above `tol`),
    accept lengths and emitted tokens bit for bit.  Returns (baseline, parity).
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import accept_greedy, accept_stochastic, verify_attention_unit

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:        # pragma: no cover
        threadpool_limits = None
    sp = inp.spec
    B, Hkv, G = sp.batch, sp.kv_heads, sp.group
    usable, host_cpus, model = cpu_info()
    workers = max(1, min(ORACLE_THREADS, usable))
    rng = np.random.default_rng(1)

    def bits(t):
        import torch
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    qs = inp.q_start.cpu().numpy()
    kvl = inp.kv_len.cpu().numpy()
    v_layout = "key" if tuple(inp.v_cache.shape) == tuple(inp.k_cache.shape) else "dim"
    seq_cache = {}
    got = gpu_out.float().cpu().numpy() if gpu_out is not None else None
    att_err, att_over, att_units, att_nonfinite = 0.0, 0, 0, 0

    def seq_args(b):
        # host copy of one sequence's pages, shared by its KV heads
        if b not in seq_cache:
            n = int(kvl[b])
            npg = (n + sp.page_size - 1) // sp.page_size
            pages = inp.block_table[b, :npg].long()
            t0, t1 = int(qs[b]), int(qs[b + 1])
            seq_cache[b] = dict(q_bits=bits(inp.q[t0:t1]), k_bits=bits(inp.k_cache[pages]),
                                v_bits=bits(inp.v_cache[pages]), block_table=np.arange(npg, dtype=np.int32)[None],
                                kv_len=np.asarray([n], np.int32), q_start=np.asarray([0, t1 - t0], np.int32),
                                group=G, b=0, v_layout=v_layout)
        return seq_cache[b]

    order = [(int(b), h) for b in rng.permutation(B) for h in range(Hkv)]
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t_attn, done = 0.0, 0
        with ThreadPoolExecutor(workers) as ex:
            for i in range(0, len(order), workers):
                batch = order[i:i + workers]
                args = [dict(seq_args(b), h=h) for b, h in batch]
                t_start = time.perf_counter()
                refs = list(ex.map(lambda a: verify_attention_unit(**a), args))
                t_attn += time.perf_counter() - t_start
                done += len(batch)
                if got is not None:
                    for (b, h), ref in zip(batch, refs):
                        g = got[int(qs[b]):int(qs[b + 1]), h * G:(h + 1) * G]
                        fin = np.isfinite(g)
                        att_nonfinite += int((~fin).sum())
                        e = np.abs(np.where(fin, g, 0.0) - ref)
                        att_err = max(att_err, float(e.max()) if e.size else 0.0)
                        att_over += int((e > tol).sum()) + int((~fin).sum())
                        att_units += 1
                for b, _ in batch:
                    if all(o[0] != b for o in order[i + workers:]):
                        seq_cache.pop(b, None)
                if t_attn > budget_s:
                    break
        seq_cache.clear()
        tl = inp.target_logits
        dl = inp.draft_logits
        toks = inp.draft_tokens.cpu().numpy()
        uni = inp.uniforms.cpu().numpy()
        al_gpu = gpu_al.cpu().numpy() if gpu_al is not None else None
        tok_gpu = gpu_tok.cpu().numpy() if gpu_tok is not None else None
        acc_seqs, al_bad, tok_bad = 0, 0, 0
        t_acc, done_acc = 0.0, 0
        seqs = [int(b) for b in rng.permutation(B)]
        with ThreadPoolExecutor(workers) as ex:
            for i in range(0, B, workers):
                jobs, bs = [], seqs[i:i + workers]
                for b in bs:
                    t0, t1 = int(qs[b]), int(qs[b + 1])
                    d0 = t0 - b
                    job = dict(target_logits=tl[t0:t1].cpu().numpy(), draft_tokens=toks[d0:d0 + t1 - t0 - 1],
                               q_start=np.asarray([0, t1 - t0], np.int32))
                    if sp.mode == "stochastic":
                        job.update(draft_logits=dl[d0:d0 + t1 - t0 - 1].cpu().numpy(), uniforms=uni[t0:t1])
                    jobs.append(job)
                t_start = time.perf_counter()
                if sp.mode == "stochastic":
                    res = list(ex.map(lambda j: accept_stochastic(**j), jobs))
                else:
                    res = list(ex.map(lambda j: accept_greedy(j["target_logits"], j["draft_tokens"], j["q_start"]),
                                      jobs))
                t_acc += time.perf_counter() - t_start
                done_acc += len(jobs)
                if al_gpu is not None:
                    for b, (al_o, tok_o) in zip(bs, res):
                        t0, t1 = int(qs[b]), int(qs[b + 1])
                        acc_seqs += 1
                        al_bad += int(al_o[0] != al_gpu[b])
                        tok_bad += int(not np.array_equal(tok_o, tok_gpu[t0:t1]))
                if t_acc > budget_s / 2:
                    break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    step_s = t_attn * (B * Hkv) / done + t_acc * B / done_acc
    T = int(qs[-1])
    whole = done == B * Hkv and done_acc == B
    used = max(min(workers, B * Hkv), min(workers, B))   # threads the pools actually ran
    base = {"value": T / step_s, "unit": "verified tokens/s", "cores": used, "kind": "oracle",
            "sample": (f"{done} of {B * Hkv} (sequence, KV head) attention units and {done_acc} of {B} sequences' "
                       f"accept/reject, fp64 oracle on {used} threads"
                       + ("" if whole else ", scaled to the whole step")),
            "step_seconds_estimate": step_s, "sample_seconds": t_attn + t_acc,
            "host_cpus": host_cpus, "usable_cpus": usable, "cpu_model": model}
    parity = None
    if got is not None:
        parity = {"attention": {"units_compared": att_units, "units_total": B * Hkv, "max_abs_err": att_err,
                                "elements_over_tol": att_over, "non_finite": att_nonfinite, "tol": tol},
                  "accept": {"sequences_compared": acc_seqs, "sequences_total": B,
                             "accept_len_mismatches": al_bad, "token_mismatches": tok_bad},
                  "ok": att_over == 0 and al_bad == 0 and tok_bad == 0 and att_units > 0 and acc_seqs > 0}
    return base, parity


def attention_source_digest() -> str:
    """sha256 of the attention kernels' source: a stored traffic figure is used
    only while the kernel it was measured on is unchanged."""
    import hashlib
    path = os.path.join(ROOT, "speculative_decoding_verification_sd_amd", "csrc", "attention.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per launch of the dominant attention kernel for `workload`,
    from the counter summary under profiles/ (FETCH_SIZE + WRITE_SIZE, scaled
    by a plain copy's reading), or None when there is none for the current
    kernel source."""
    path = os.path.join(ROOT, "profiles", f"verify_attn_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#", "$")):
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("attention_source_sha256") != attention_source_digest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _rocprof_csv(d: str, kind: str):
    import csv
    import glob
    hits = glob.glob(os.path.join(d, f"*{kind}.csv"))
    if not hits:
        raise SystemExit(f"no *{kind}.csv under {d}")
    with open(hits[0]) as f:
        return list(csv.DictReader(f))


def _per_dispatch(d: str):
    """{dispatch id: (kernel name, summed counter value)} of one rocprofv3 --pmc run."""
    per = {}
    for r in _rocprof_csv(d, "counter_collection"):
        name, v = per.get(r["Dispatch_Id"], (r["Kernel_Name"], 0.0))
        per[r["Dispatch_Id"]] = (name, v + float(r["Counter_Value"]))
    return per


def workload_args(cfg) -> str:
    """The bench.py options that select the workload of a bench line's config."""
    from workloads import PRESETS
    wl = cfg["workload"]
    for key, v in PRESETS.items():
        if v.name == wl:
            return "" if key == "g8_kv32k_D15" else f" --workload {key}"
        if v.name.endswith("_sweep") and v.name.replace("_sweep", f"_D{cfg.get('draft_len')}") == wl:
            return f" --workload {key} --draft {cfg['draft_len']}"
    raise SystemExit(f"workload {wl} is not a preset")


def write_bench_lines(*bench_jsons):
    """profiles/ table of bench lines (one per workload, each with its oracle
    baseline and parity), followed by the lines themselves and their commands."""
    rows, body = [], []
    for path in bench_jsons:
        with open(path) as f:
            line = json.loads(f.read().strip().splitlines()[-1])
        cfg, r, c, pa = line["config"], line["roofline"], line["cpu_baseline"], line["parity"]["attention"]
        rows.append(f"{cfg['workload'][:52]:52s} {line['value']:10.4g} {line['step_us']:8.1f} "
                    f"{line['attention_ms'] * 1e3:8.1f} {line['accept_ms'] * 1e3:7.1f} {r['frac']:6.3f} "
                    f"{r['mfma_frac']:6.3f} {c['value']:10.4g} "
                    f"{str(pa['units_compared']) + '/' + str(pa['units_total']):>12s} {pa['max_abs_err']:9.2e} "
                    f"{str(line['parity']['ok']):>6s}")
        body += [f"$ python3 REPO/bench.py{workload_args(cfg)}", json.dumps(line), ""]
    path = os.path.join(ROOT, "profiles", "verify_step_bench_lines_all_workloads.txt")
    with open(path, "w") as f:
        f.write("# bench.py lines of every workload (one MI355X, inputs resident in HBM, median of the timed steps\n"
                "# (\"steps\" in each line), 1 GiB cache flush before each step outside the timed events), each with\n"
                "# its oracle baseline on the box's 16-core host share and the element-by-element parity of the\n"
                "# oracle units it ran against the GPU outputs of the same call.  hbm / mfma: algorithmic attention bytes / flops over\n"
                "# the whole attention call (plan + main + combine) against 8 TB/s and 2.5 PFLOP/s bf16.\n\n")
        f.write(f"{'workload':52s} {'tok/s':>10s} {'step_us':>8s} {'attn_us':>8s} {'acc_us':>7s} {'hbm':>6s} "
                f"{'mfma':>6s} {'cpu tok/s':>10s} {'units':>12s} {'max_err':>9s} {'parity':>6s}\n")
        f.write("\n".join(rows) + "\n\n" + "\n".join(body))
    print(f"wrote {path}")


def write_profiles(bench_json: str, kt_dir: str, fetch_dir: str, write_dir: str, copy_bytes: int):
    """Write the kernel-time and HBM-traffic summaries under profiles/ from one
    bench.py JSON line and three rocprofv3 runs of bench.py (kernel trace with
    --stats, FETCH_SIZE pass, WRITE_SIZE pass; the counter passes ran with
    --calibrate-copy `copy_bytes`)."""
    import statistics
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    cfg = line["config"]
    wl = cfg["workload"]
    args = "--no-cpu-baseline" + workload_args(cfg)
    # kernel-time summary: the library's kernels only
    stats = [r for r in _rocprof_csv(kt_dir, "kernel_stats") if "sdv::" in r["Name"]]
    calls = int(stats[0]["Calls"]) if stats else 0
    main = max((r for r in stats if "verify_attn" in r["Name"]), key=lambda r: float(r["TotalDurationNs"]))
    prof = os.path.join(ROOT, "profiles")
    with open(os.path.join(prof, f"verify_step_{wl}_kernel_stats.txt"), "w") as f:
        f.write(f"# rocprofv3 kernel-trace summary of the library's kernels, workload {wl}:\n"
                "# one verify step = verify attention (plan, main, split-KV combine) + accept/reject.\n"
                f"# {calls} calls per kernel = clock-settle + warmup + timed steps.  Durations in ns.\n"
                f"$ cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d OUT/kt "
                f"-o run --output-format csv -- python3 REPO/bench.py {args}\n")
        f.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n")
        for r in stats:
            f.write(",".join([r["Name"], r["Calls"], r["TotalDurationNs"], r["AverageNs"], r["Percentage"],
                              r["MinNs"], r["MaxNs"], r["StdDev"]]) + "\n")
        attn = sum(float(r["AverageNs"]) for r in stats if "verify_attn" in r["Name"]) / 1e3
        f.write(f"attention call (plan + main + combine averages): {attn:.1f} us\n")
        f.write(f"bench.py in the same call: attention {line['attention_ms'] * 1e3:.1f} us/step (HIP events), "
                f"accept {line['accept_ms'] * 1e3:.1f} us/step, {line['value']:.0f} verified tokens/s\n")
    # traffic summary of the dominant kernel
    kname = main["Name"]
    fetch, write = _per_dispatch(fetch_dir), _per_dispatch(write_dir)
    fk = statistics.median(v for n, v in fetch.values() if n == kname)
    wk = statistics.median(v for n, v in write.values() if n == kname)
    nk = sum(1 for n, _ in fetch.values() if n == kname)
    copy_w = [v for n, v in write.values() if "copyBuffer" in n and abs(v * 1024 - copy_bytes) < 1024]
    copy_f = sorted((v for n, v in fetch.values() if "copyBuffer" in n), reverse=True)[:len(copy_w)]
    if not copy_w or not copy_f:
        raise SystemExit("no calibration copy found in the counter runs")
    cw, cf = statistics.median(copy_w), statistics.median(copy_f)
    fscale, wscale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    hbm = fk * 1024 * fscale + wk * 1024 * wscale
    alg = line["roofline"]["algorithmic_bytes_per_launch"]
    short = kname.replace("void ", "").split("(")[0].replace("sdv::", "")
    with open(os.path.join(prof, f"verify_attn_traffic_{wl}.txt"), "w") as f:
        f.write(f"# HBM traffic per launch of the dominant kernel ({short}) on workload {wl}, from two\n"
                f"# rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, median of {nk}\n"
                f"# launches).  Each pass also runs a plain {copy_bytes >> 20} MiB device-to-device copy\n"
                "# (__amd_rocclr_copyBuffer) whose counter readings give the scale from counter KiB to bytes.\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            f.write(f"$ cd /tmp && export TMPDIR=/tmp && timeout -s KILL 90 rocprofv3 --pmc {c} --kernel-trace "
                    f"-d OUT/pmc_{c.split('_')[0].lower()} -o run --output-format csv -- python3 "
                    f"REPO/bench.py {args} --settle-s 0 --steps 5 --warmup 2 --calibrate-copy {copy_bytes}\n")
        f.write(f"kernel: {short}\n"
                f"attention_source_sha256: {attention_source_digest()}\n"
                f"fetch_kib_per_launch: {fk:.1f}\nwrite_kib_per_launch: {wk:.1f}\n"
                f"copy_bytes: {copy_bytes}\ncopy_fetch_kib: {cf:.1f}\ncopy_write_kib: {cw:.1f}\n"
                f"fetch_scale: {fscale:.5f}\nwrite_scale: {wscale:.5f}\n"
                f"hbm_bytes_per_launch: {hbm:.0f}\nalgorithmic_bytes_per_launch: {alg}\n"
                f"traffic_over_algorithmic: {hbm / alg:.4f}\n"
                f"kernel_average_ns (kernel trace): {float(main['AverageNs']):.0f}\n")
    print(f"wrote profiles for {wl}: {short} {float(main['AverageNs']) / 1e3:.1f} us, traffic {hbm / alg:.4f}x")


# Counter passes of the attention's dominant kernel (one rocprofv3 --pmc run each; at most 8 SQ counters).
COUNTER_PASSES = [
    "GRBM_GUI_ACTIVE SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
    "SQ_INSTS_VALU_TRANS_F32",
    "GRBM_GUI_ACTIVE SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS "
    "SQ_WAVE_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES",
    "GRBM_GUI_ACTIVE SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INST_CYCLES_SALU SQ_INSTS_SALU "
    "SQ_ACTIVE_INST_ANY SQ_LDS_DATA_FIFO_FULL",
]
XCDS, CUS, SIMDS = 8, 256, 1024       # MI355X: GRBM_GUI_ACTIVE sums the XCDs' busy cycles


def write_counter_profile(label: str, args_str: str, *pass_dirs):
    """Per-launch counter summary of the dominant attention kernel under
    profiles/, from the rocprofv3 --pmc runs of COUNTER_PASSES (medians over the
    launches), with the derived clock, MFMA busy fraction, LDS activity and
    MFMA/VALU co-execution."""
    import statistics
    from collections import defaultdict
    vals, durs, kname = {}, [], None
    for d in pass_dirs:
        per, ts = defaultdict(dict), {}
        for r in _rocprof_csv(d, "counter_collection"):
            if "verify_attn" not in r["Kernel_Name"]:
                continue
            kname = r["Kernel_Name"]
            per[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
            ts[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for k in {k for v in per.values() for k in v}:
            vals.setdefault(k, []).append(statistics.median(v[k] for v in per.values() if k in v))
        durs += list(ts.values())
    c = {k: statistics.mean(v) for k, v in vals.items()}
    dur = statistics.median(durs) * 1e-9
    cyc = c["GRBM_GUI_ACTIVE"] / XCDS
    short = kname.replace("void ", "").split("(")[0].replace("sdv::", "")
    path = os.path.join(ROOT, "profiles", f"verify_attn_counters_{label}.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 counters of {short} on workload {label}: medians per launch over the launches of\n"
                f"# each pass ({len(pass_dirs)} passes, one rocprofv3 run each).  Launches run one at a time under\n"
                "# counter collection, so the clock here can differ from back-to-back runs.\n")
        for i, d in enumerate(pass_dirs):
            f.write(f"$ cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc {COUNTER_PASSES[i]} "
                    f"--kernel-include-regex verify_attn_wide -d OUT/pmc_p{i + 1} -o run --output-format csv -- "
                    f"python3 REPO/bench.py --no-cpu-baseline --settle-s 0 --steps 3 --warmup 1 {args_str}\n")
        f.write(f"kernel: {short}\nkernel_us: {dur * 1e6:.1f}\n")
        for k in sorted(c):
            f.write(f"{k}: {c[k]:.6g}\n")
        mfma = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * SIMDS)
        f.write("# derived (per-XCD cycles = GRBM_GUI_ACTIVE / 8; 1024 SIMDs, 256 CUs)\n")
        f.write(f"clock_ghz: {cyc / dur / 1e9:.3f}\n")
        f.write(f"mfma_busy_frac_of_cycles: {mfma:.3f}\n")
        f.write(f"mfma_busy_frac_of_2.4GHz_peak: {mfma * cyc / dur / 2.4e9:.3f}\n")
        f.write(f"mfma_valu_coexec_frac: {c.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0) / (cyc * SIMDS):.3f}\n")
        f.write(f"lds_idx_active_frac: {c.get('SQ_LDS_IDX_ACTIVE', 0.0) / (cyc * CUS):.3f}\n")
        f.write(f"lds_bank_conflict_cycles: {c.get('SQ_LDS_BANK_CONFLICT', 0.0):.0f}\n")
        waves = c.get("SQ_WAVES", 1.0)
        for k in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            f.write(f"{k.lower()}_per_wave: {c.get(k, 0.0) / waves:.0f}\n")
        if "SQ_WAVE_CYCLES" in c:
            f.write(f"wait_any_per_wave_cycle: {c.get('SQ_WAIT_ANY', 0.0) / c['SQ_WAVE_CYCLES']:.3f}\n")
            f.write(f"valu_active_per_wave_cycle: {c.get('SQ_ACTIVE_INST_VALU', 0.0) / c['SQ_WAVE_CYCLES']:.3f}\n")
        f.write(f"bf16_mfma_flops (MOPS x 512): {c.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0.0) * 512:.4g}\n")
    print(f"wrote {path}")


SWEEP_PRESET = "g8_kv32k_sweep"
TREE_PRESET = "g8_kv32k_D15"
TREE_BRANCHING = (2, 2, 2, 2)   # a full binary tree of depth 4: 30 drafted nodes, G*(1+30) = 248 rows


def tree_algorithmic(inp, parents):
    """Bytes and flops of one tree-attention call: every key read once; node i of
    sequence b sees the N_b-1-T_b prefix keys plus the nodes on its root path."""
    import numpy as np
    kv = inp.kv_len.cpu().numpy().astype(np.int64)
    qs = inp.q_start.cpu().numpy().astype(np.int64)
    par = parents.cpu().numpy().astype(np.int64)
    sp = inp.spec
    d, Hkv, G = sp.head_dim, sp.kv_heads, sp.group
    T_q = int(qs[-1])
    nbytes = int((kv * Hkv * d * 2 * 2).sum()) + 2 * T_q * Hkv * G * d * 2 \
        + int(((kv + sp.page_size - 1) // sp.page_size).sum()) * 4 + par.size * 4 + T_q * 8
    visible = 0
    for b in range(len(kv)):
        T = int(qs[b + 1] - qs[b]) - 1
        depth = [0] * (T + 1)
        for i in range(1, T + 1):
            depth[i] = depth[int(par[qs[b] - b + i - 1])] + 1
        visible += sum(max(int(kv[b]) - 1 - T, 0) + depth[i] + 1 for i in range(T + 1))
    return nbytes, 4 * d * Hkv * G * visible


def run_tree(args):
    """Tree verification (ancestor-mask attention + greedy longest-path
    acceptance) on the default shapes with a full binary draft tree of depth 4;
    one JSON line."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv
    from workloads import preset
    from workloads.tree import tree_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sp = preset(TREE_PRESET, seed=args.seed, v_layout=args.v_layout)
    print(f"[bench] tree {TREE_BRANCHING}: generating", file=sys.stderr, flush=True)
    inp, parents, tokens = tree_inputs(sp, TREE_BRANCHING, device=dev)
    B, T_q = sp.batch, inp.q.shape[0]
    out = torch.empty_like(inp.q)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(T_q, dtype=torch.int32, device=dev)
    nodes = torch.empty(T_q, dtype=torch.int32, device=dev)
    adesc = sdv.attn_desc(inp.q, inp.k_cache, inp.block_table, sp.group, inp.max_draft)
    cdesc = sdv.accept_desc(B, sp.vocab, inp.max_draft, "greedy")
    ws_a = torch.empty(max(1, sdv.sd_verify_attention_workspace_size(adesc, T_q)), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, sdv.sd_tree_accept_workspace_size(cdesc, T_q)), dtype=torch.uint8, device=dev)

    def attention():
        sdv.sd_verify_tree_attention(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start,
                                     parents, out, group_size=sp.group, max_draft=inp.max_draft, workspace=ws_a)

    def accept():
        sdv.sd_tree_accept(inp.target_logits, tokens, inp.q_start, parents, al, tok, nodes,
                           max_draft=inp.max_draft, workspace=ws_c)

    t_end = time.perf_counter() + max(0.0, args.settle_s)
    while time.perf_counter() < t_end:
        for _ in range(5):
            attention()
            accept()
        torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):
        attention()
        accept()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        attention()
        ev[k][1].record(stream)
        accept()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    a_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    c_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    a_bytes, a_flops = tree_algorithmic(inp, parents)
    c_bytes = T_q * sp.vocab * 4
    step_s = (a_ms + c_ms) * 1e-3
    achieved = a_bytes / (a_ms * 1e-3) / 1e9
    ntree = len(parents) // B
    print(json.dumps({
        "metric": "draft-tree nodes verified/s per tree-verify step (+ % HBM roofline of the tree attention)",
        "value": T_q / step_s, "unit": "tree nodes/s", "higher_is_better": True, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": a_ms + c_ms, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{sp.name.replace('_D15', '')}_tree{''.join(map(str, TREE_BRANCHING))}_greedy",
                   "batch": B, "kv_heads": sp.kv_heads, "group": sp.group, "head_dim": sp.head_dim,
                   "kv_len": sp.kv_len, "vocab": sp.vocab, "tree_branching": list(TREE_BRANCHING),
                   "tree_nodes": ntree + 1, "rows_per_kv_head": sp.group * (ntree + 1), "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "tree verify attention (masks + plan + main + combine launches)",
                     "algorithmic_bytes_per_launch": a_bytes,
                     "mfma_tflops": a_flops / (a_ms * 1e-3) / 1e12,
                     "mfma_frac": a_flops / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "attention_ms": a_ms, "accept_ms": c_ms, "accept_gbs": c_bytes / (c_ms * 1e-3) / 1e9,
        "mean_accept_len": float(al.float().mean().item()),
        "accepted_tokens_per_s": float(al.sum().item()) / step_s,
        "clock_settle_s": args.settle_s}), flush=True)


def run_lossy(args):
    """Relaxed acceptance (a draft also passes when the JS distance of its rows
    is at most tau) on the default workload, timed beside the lossless call and
    the attention; one JSON line."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv
    from workloads import generate, preset

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sp = preset("g8_kv32k_D15", seed=args.seed, v_layout=args.v_layout)
    tau = args.js_threshold
    print(f"[bench] lossy tau={tau}: generating {sp.name}", file=sys.stderr, flush=True)
    inp = generate(sp, device=dev)
    B, T, V = sp.batch, inp.q.shape[0], sp.vocab
    out = torch.empty_like(inp.q)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    al0 = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(T, dtype=torch.int32, device=dev)
    ent = torch.empty(T - B, dtype=torch.float32, device=dev)
    js = torch.empty(T - B, dtype=torch.float32, device=dev)
    adesc = sdv.attn_desc(inp.q, inp.k_cache, inp.block_table, sp.group, inp.max_draft)
    cdesc = sdv.accept_desc(B, V, inp.max_draft, sp.mode)
    ws_a = torch.empty(max(1, sdv.sd_verify_attention_workspace_size(adesc, T)), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, sdv.sd_accept_lossy_workspace_size(cdesc, T)), dtype=torch.uint8, device=dev)

    def attention():
        sdv.sd_verify_attention(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start, out,
                                group_size=sp.group, max_draft=inp.max_draft, workspace=ws_a)

    def lossless():
        sdv.sd_accept_reject(inp.target_logits, inp.draft_logits, inp.draft_tokens, inp.q_start, inp.uniforms,
                             al0, tok, mode=sp.mode, max_draft=inp.max_draft, workspace=ws_c)

    def lossy():
        sdv.sd_accept_lossy(inp.target_logits, inp.draft_logits, inp.draft_tokens, inp.q_start, inp.uniforms,
                            al, tok, mode=sp.mode, max_draft=inp.max_draft, js_threshold=tau,
                            draft_entropy=ent, js_distance=js, workspace=ws_c)

    t_end = time.perf_counter() + max(0.0, args.settle_s)
    while time.perf_counter() < t_end:
        for _ in range(5):
            attention()
            lossless()
            lossy()
        torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):
        attention()
        lossless()
        lossy()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        attention()
        ev[k][1].record(stream)
        lossless()
        ev[k][2].record(stream)
        lossy()
        ev[k][3].record(stream)
    torch.cuda.synchronize()
    a_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    l0_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    l_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    c0 = algorithmic_accept(inp)
    c_bytes = c0 + 2 * (T - B) * V * 4          # + the second read of every drafted row pair
    achieved = c_bytes / (l_ms * 1e-3) / 1e9
    step_s = (a_ms + l_ms) * 1e-3
    print(json.dumps({
        "metric": "verified tokens/s per verify step with JS-relaxed acceptance (+ % HBM roofline of the "
                  "relaxed accept call)",
        "value": T / step_s, "unit": "verified tokens/s", "higher_is_better": True, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": a_ms + l_ms, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": f"{sp.name}_lossy", "batch": B, "kv_heads": sp.kv_heads, "group": sp.group,
                   "head_dim": sp.head_dim, "kv_len": sp.kv_len, "draft_len": sp.draft_len, "vocab": V,
                   "accept": sp.mode, "js_threshold": tau, "seed": sp.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "relaxed accept/reject (row statistics, JS terms, decision and sampling launches)",
                     "algorithmic_bytes_per_launch": c_bytes},
        "attention_ms": a_ms, "lossless_accept_ms": l0_ms, "lossy_accept_ms": l_ms,
        "mean_accept_len": float(al.float().mean().item()),
        "mean_accept_len_lossless": float(al0.float().mean().item()),
        "emitted_tokens_per_s": float(al.sum().item()) / step_s,
        "emitted_tokens_per_s_lossless": float(al0.sum().item()) / ((a_ms + l0_ms) * 1e-3),
        "mean_js_distance": float(js.mean().item()), "mean_draft_entropy": float(ent.mean().item()),
        "clock_settle_s": args.settle_s}), flush=True)


def run_read_ceiling(args):
    """The HBM read rate a plain library reduction reaches on this GPU (row sums
    of a 2 GiB fp32 matrix of 4096-wide rows, cold each time), as the practical
    read ceiling next to the datasheet peak; one JSON line."""
    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nbytes = 2 << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev).view(-1, 4096)
    other = torch.ones(nbytes // 4, dtype=torch.float32, device=dev).view(-1, 4096)   # evicts x between runs
    sink = torch.empty(x.shape[0], dtype=torch.float32, device=dev)
    times = []
    for k in range(args.warmup + args.steps):
        torch.sum(other, dim=1, out=sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.sum(x, dim=1, out=sink)
        e1.record()
        torch.cuda.synchronize()
        if k >= args.warmup:
            times.append(e0.elapsed_time(e1) * 1e-3)
    t = float(np.median(times))
    print(json.dumps({"metric": "HBM read rate of a plain reduction (practical read ceiling)",
                      "value": nbytes / t / 1e9, "unit": "GB/s", "peak": HBM_PEAK_GBS,
                      "frac": nbytes / t / 1e9 / HBM_PEAK_GBS, "bytes": nbytes, "us": t * 1e6,
                      "kernel": "torch.sum over the rows of a 2 GiB fp32 [131072, 4096] matrix",
                      "steps": args.steps}), flush=True)


LOOP_B, LOOP_V, LOOP_PROMPT, LOOP_MAX_LEN, LOOP_STEPS = 64, 4096, 256, 4096, 400


def run_loop(args):
    """The closed speculative-decoding loop on a bigram toy LM (64 sequences,
    V = 4096, 256-token random prompts, trigram drafter), adaptive over tiers
    1/3/7 with one graph per tier, beside the same loop with direct launches,
    a fixed top tier and no speculation (D = 0); one JSON line."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator().manual_seed(args.seed)
    W = (torch.randn((LOOP_V, LOOP_V), generator=g) * 3.0).to(dev)
    rng = np.random.default_rng(args.seed)
    prompts = torch.from_numpy(rng.integers(0, LOOP_V, size=(LOOP_B, LOOP_PROMPT)).astype(np.int32))
    ws = torch.empty(sdv.sd_closed_loop_workspace_size(sdv.loop_desc(LOOP_B, LOOP_V, LOOP_MAX_LEN, (0, 1, 3, 7))),
                     dtype=torch.uint8, device=dev)

    def once(tiers, graphs, steps=LOOP_STEPS):
        h = torch.zeros((LOOP_B, LOOP_MAX_LEN), dtype=torch.int32, device=dev)
        h[:, :LOOP_PROMPT] = prompts.to(dev)
        ln = torch.full((LOOP_B,), LOOP_PROMPT, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        t = time.perf_counter()
        al, tr = sdv.sd_closed_loop(W, h, ln, steps=steps, tiers=tiers, ngram=3, ema_weight=0.5,
                                    use_graphs=graphs, workspace=ws)
        torch.cuda.synchronize()
        t = time.perf_counter() - t
        return t, al.numpy(), tr.numpy(), (h.cpu().numpy(), ln.cpu().numpy())

    once((1, 3, 7), True, steps=20)                          # warm the clock and the code paths
    runs, outs = {}, []
    for name, tiers, graphs in (("adaptive_graphs", (1, 3, 7), True), ("adaptive_direct", (1, 3, 7), False),
                                ("fixed_D7_graphs", (7,), True), ("no_speculation_graphs", (0,), True)):
        t, al, tr, h = once(tiers, graphs)
        runs[name] = {"seconds": t, "tokens": int(al.sum()), "tokens_per_s": float(al.sum()) / t,
                      "us_per_round": t / LOOP_STEPS * 1e6, "mean_al": float(al[al > 0].mean()),
                      "rounds_per_tier": {str(d): int((tr == d).sum()) for d in sorted(set(tr.tolist()))}}
        print(f"[bench] loop {name}: {runs[name]['tokens_per_s']:.0f} tok/s, {runs[name]['us_per_round']:.1f} "
              f"us/round, AL {runs[name]['mean_al']:.2f}", file=sys.stderr, flush=True)
        outs.append(h)
    # every run is the same greedy decoding, so the histories agree on their common prefix
    agree = all(np.array_equal(a[0][b, :min(a[1][b], c[1][b])], c[0][b, :min(a[1][b], c[1][b])])
                for a in outs for c in outs for b in range(LOOP_B))
    main = runs["adaptive_graphs"]
    # per-round algorithmic bytes: W rows gathered into the logits (read + write) and read once by the accept
    # pass, at the adaptive run's mean 1+D
    rows = LOOP_B * (1 + np.mean([int(d) for d, n in main["rounds_per_tier"].items() for _ in range(n)]))
    nbytes = rows * LOOP_V * 4 * 3
    achieved = nbytes / (main["us_per_round"] * 1e-6) / 1e9
    print(json.dumps({
        "metric": "emitted tokens/s of the closed adaptive speculative-decoding loop (bigram toy LM)",
        "value": main["tokens_per_s"], "unit": "emitted tokens/s", "higher_is_better": True, "n_gpus": 1,
        "steps": LOOP_STEPS, "warmup": 20, "ms_per_step": main["us_per_round"] / 1e3, "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"loop_b{LOOP_B}_v{LOOP_V}_prompt{LOOP_PROMPT}_tiers137_ngram3", "batch": LOOP_B,
                   "vocab": LOOP_V, "prompt": LOOP_PROMPT, "max_len": LOOP_MAX_LEN, "rounds": LOOP_STEPS,
                   "tiers": [1, 3, 7], "ngram": 3, "ema_weight": 0.5, "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "one round (draft, toy-LM logits, accept, append) incl. launch and host sync",
                     "algorithmic_bytes_per_launch": nbytes,
                     "note": "latency-bound: a round moves a few MB and waits for the host each time"},
        "outputs_agree": bool(agree), "runs": runs}), flush=True)


def write_loop_profile(bench_json: str, kt_dir: str):
    """Kernel-time summary under profiles/ of a rocprofv3 --kernel-trace --stats
    run of `bench.py --loop`, with the bench line of the same call."""
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    wl = line["config"]["workload"]
    stats = [r for r in _rocprof_csv(kt_dir, "kernel_stats") if "sdv::" in r["Name"]]
    path = os.path.join(ROOT, "profiles", f"closed_loop_{wl}_kernel_stats.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel-trace summary of the closed loop, workload {wl}: every round runs\n"
                "# loop_draft, loop_logits, accept_rowstats<0,...>, accept_decide<false>, loop_append; the calls\n"
                "# cover all four runs of bench.py --loop (adaptive with graphs, adaptive with direct launches,\n"
                "# fixed D = 7, no speculation) and the warm-up.  Durations in ns.\n"
                "$ cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d OUT/kt_loop "
                "-o run --output-format csv -- python3 REPO/bench.py --loop\n")
        f.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n")
        for r in stats:
            f.write(",".join([r["Name"], r["Calls"], r["TotalDurationNs"], r["AverageNs"], r["Percentage"],
                              r["MinNs"], r["MaxNs"], r["StdDev"]]) + "\n")
        per_round = sum(float(r["AverageNs"]) for r in stats if "qstart" not in r["Name"])
        f.write(f"kernel time per round (sum of the five averages): {per_round / 1e3:.1f} us\n")
        for name, r in line["runs"].items():
            f.write(f"bench.py {name}: {r['us_per_round']:.1f} us/round wall (incl. launch and host sync), "
                    f"{r['tokens_per_s']:.0f} emitted tokens/s, mean AL {r['mean_al']:.2f}\n")
    print(f"wrote {path}")


def write_lossy_profile(bench_json: str, kt_dir: str):
    """Kernel-time summary under profiles/ of a rocprofv3 --kernel-trace --stats
    run of `bench.py --lossy`, with the bench line of the same call."""
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    wl = line["config"]["workload"]
    stats = [r for r in _rocprof_csv(kt_dir, "kernel_stats") if "sdv::" in r["Name"] and "attn" not in r["Name"]]
    path = os.path.join(ROOT, "profiles", f"accept_lossy_{wl}_kernel_stats.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel-trace summary of the accept kernels, workload {wl} (tau = "
                f"{line['config']['js_threshold']}):\n"
                "# each step runs the lossless call (accept_rowstats<1,...>, accept_finish<false>, accept_draw) and\n"
                "# the relaxed call (accept_rowstats<3,...>, accept_jsd, accept_finish<true>, accept_draw; the draw\n"
                "# kernel is the same in both, so its line counts two launches per step).  Calls = clock-settle +\n"
                "# warmup + timed steps.  Durations in ns.\n"
                "$ cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d OUT/kt_lossy "
                "-o run --output-format csv -- python3 REPO/bench.py --lossy\n")
        f.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n")
        for r in stats:
            f.write(",".join([r["Name"], r["Calls"], r["TotalDurationNs"], r["AverageNs"], r["Percentage"],
                              r["MinNs"], r["MaxNs"], r["StdDev"]]) + "\n")
        lossy = sum(float(r["AverageNs"]) for r in stats if "rowstats<3" in r["Name"] or "jsd" in r["Name"]
                    or "finish<true>" in r["Name"] or "accept_draw" in r["Name"])
        f.write(f"relaxed accept call (rowstats<3> + jsd + finish<true> + draw averages): {lossy / 1e3:.1f} us\n")
        f.write(f"bench.py in the same call: relaxed accept {line['lossy_accept_ms'] * 1e3:.1f} us/step, lossless "
                f"{line['lossless_accept_ms'] * 1e3:.1f} us/step (HIP events), HBM {line['roofline']['frac']:.3f} "
                f"of peak, mean AL {line['mean_accept_len']:.3f} (lossless {line['mean_accept_len_lossless']:.3f})\n")
    print(f"wrote {path}")


def write_tree_profile(bench_json: str, kt_dir: str):
    """Kernel-time summary under profiles/ of a rocprofv3 --kernel-trace --stats
    run of `bench.py --tree`, with the bench line of the same call."""
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    wl = line["config"]["workload"]
    stats = [r for r in _rocprof_csv(kt_dir, "kernel_stats") if "sdv::" in r["Name"]]
    calls = int(stats[0]["Calls"]) if stats else 0
    path = os.path.join(ROOT, "profiles", f"verify_tree_{wl}_kernel_stats.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel-trace summary of the library's kernels, workload {wl}:\n"
                "# one tree-verify step = tree attention (ancestor masks, plan, main, split-KV combine)\n"
                f"# + greedy tree acceptance (row statistics, path walk).  {calls} calls per kernel =\n"
                "# clock-settle + warmup + timed steps.  Durations in ns.\n"
                "$ cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d OUT/kt_tree "
                "-o run --output-format csv -- python3 REPO/bench.py --tree\n")
        f.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n")
        for r in stats:
            f.write(",".join([r["Name"], r["Calls"], r["TotalDurationNs"], r["AverageNs"], r["Percentage"],
                              r["MinNs"], r["MaxNs"], r["StdDev"]]) + "\n")
        attn = sum(float(r["AverageNs"]) for r in stats if "verify_attn" in r["Name"] or "tree_masks" in r["Name"])
        f.write(f"tree attention call (masks + plan + main + combine averages): {attn / 1e3:.1f} us\n")
        f.write(f"bench.py in the same call: attention {line['attention_ms'] * 1e3:.1f} us/step (HIP events), "
                f"accept {line['accept_ms'] * 1e3:.1f} us/step, {line['value']:.0f} tree nodes/s, "
                f"HBM {line['roofline']['frac']:.3f} of peak, mean AL {line['mean_accept_len']:.3f}\n")
    print(f"wrote {path}")


BATCH_SWEEP = [(16, 32768), (256, 2048), (2048, 512), (4096, 256)]   # (sequences, keys each)
BATCH_SWEEP_SETTLE = 1000   # untimed calls per point before the timed ones (about a second)


def run_batch_sweep(args):
    """Verify attention time against the batch size at a fixed shape per
    sequence (H_kv=8, G=8, d=128, D=3): B sequences of N keys for the pairs of
    BATCH_SWEEP, from 16 long sequences to 4096 short ones, where the
    device-side plan and the combine cost most.  One JSON line."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv
    from workloads import WorkloadSpec, generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    points = []
    for B, N in BATCH_SWEEP:
        sp = WorkloadSpec(name=f"b{B}_hkv8_g8_d128_kv{N}_D3", batch=B, kv_heads=8, group=8, head_dim=128,
                          kv_len=N, draft_len=3, vocab=64, mode="greedy", seed=args.seed, v_layout=args.v_layout)
        print(f"[bench] batch sweep: generating {sp.name}", file=sys.stderr, flush=True)
        inp = generate(sp, device=dev)
        out = torch.empty_like(inp.q)
        desc = sdv.attn_desc(inp.q, inp.k_cache, inp.block_table, sp.group, inp.max_draft)
        ws = torch.empty(max(1, sdv.sd_verify_attention_workspace_size(desc, inp.q.shape[0])), dtype=torch.uint8,
                         device=dev)

        def attention():
            sdv.sd_verify_attention(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start,
                                    out, group_size=sp.group, max_draft=inp.max_draft, workspace=ws)

        # a fixed number of calls per point (clock settle, then the timed ones), so that
        # a kernel trace of this run splits evenly into the points
        for _ in range(BATCH_SWEEP_SETTLE):
            attention()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for k in range(args.steps):
            ev[k][0].record()
            attention()
            ev[k][1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        kv_bytes = B * N * sp.kv_heads * sp.head_dim * 4
        points.append({"batch": B, "kv_len": N, "attention_ms": ms, "hbm_frac": kv_bytes / (ms * 1e-3) / 8e12})
        del inp, out, ws
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "verify attention time against the batch size", "unit": "ms",
                      "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "dtype": "bf16",
                      "data": "synthetic", "config": {"workload": "hkv8_g8_d128_D3_batch_sweep", "seed": args.seed},
                      "points": points}))


def write_batch_profile(bench_json: str, kt_dir: str):
    """Per-kernel medians per batch point under profiles/, from a rocprofv3
    --kernel-trace run of `bench.py --batch-sweep` (the points run in order)."""
    import statistics
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    rows = [r for r in _rocprof_csv(kt_dir, "kernel_trace") if "sdv::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # every attention call has exactly one main launch (the plan may run inside it, and caches
    # that cannot be split have no combine launch): a plan or descriptor launch belongs to the
    # next main launch's call, a combine launch to the previous one's
    call_of, mains = [], 0
    for r in rows:
        name = r["Kernel_Name"]
        if "verify_attn_main" in name or "verify_attn_wide" in name:
            call_of.append(mains)
            mains += 1
        elif "verify_attn_combine" in name:
            call_of.append(mains - 1)
        else:
            call_of.append(mains)
    per_point = mains // len(line["points"])
    path = os.path.join(ROOT, "profiles", "verify_attn_batch_sweep_hkv8_g8_d128_D3.txt")
    with open(path, "w") as f:
        f.write("# Verify attention against the batch size (H_kv=8, G=8, d=128, D=3; B sequences of N keys):\n"
                "# median kernel durations per point from a rocprofv3 kernel trace, and the call time with HIP\n"
                "# events in the same run.  The plan and the combine are the launches whose cost grows with B;\n"
                "# batches of up to 32 sequences plan inside the main kernel (plan_us 0); plan_us includes the\n"
                "# descriptor kernel of batches past 4096 sequence-head pairs.\n"
                "$ cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace -d OUT/kt_batch -o run "
                "--output-format csv -- python3 REPO/bench.py --batch-sweep\n")
        f.write("batch,kv_len,plan_us,main_us,combine_us,call_us_events,hbm_frac\n")
        for k, pt in enumerate(line["points"]):
            lo, hi = k * per_point, (k + 1) * per_point
            sel = [r for r, c in zip(rows, call_of) if lo <= c < hi]
            med = {}
            for part, key in (("plan", "verify_attn_plan"), ("items", "verify_attn_items"), ("main", "verify_attn_main"),
                              ("wide", "verify_attn_wide"), ("combine", "verify_attn_combine")):
                d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel if key in r["Kernel_Name"]]
                med[part] = statistics.median(d) / 1e3 if d else 0.0
            f.write(f"{pt['batch']},{pt['kv_len']},{med['plan'] + med['items']:.1f},{med['main'] + med['wide']:.1f},"
                    f"{med['combine']:.1f},{pt['attention_ms'] * 1e3:.1f},{pt['hbm_frac']:.3f}\n")
    print(f"wrote {path}")


def run_sweep(args):
    """Verify attention (and accept) time per draft length D on the tile-boundary
    sweep workload (B=32, H_kv=8, G=8, d=128, 32768-token cache, V=32000,
    synthetic acceptance rate alpha), one JSON line with one point per D."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv
    from workloads import generate, preset

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    points = []
    alpha = args.alpha if args.alpha is not None else 0.6
    for D in args.sweep:
        sp = preset(SWEEP_PRESET, draft_len=D, alpha=alpha, seed=args.seed, v_layout=args.v_layout)
        print(f"[bench] sweep D={D}: generating {sp.name}", file=sys.stderr, flush=True)
        inp = generate(sp, device=dev)
        B, T = sp.batch, inp.q.shape[0]
        out = torch.empty_like(inp.q)
        al = torch.empty(B, dtype=torch.int32, device=dev)
        tok = torch.empty(T, dtype=torch.int32, device=dev)
        adesc = sdv.attn_desc(inp.q, inp.k_cache, inp.block_table, sp.group, inp.max_draft)
        cdesc = sdv.accept_desc(B, sp.vocab, inp.max_draft, sp.mode)
        ws_a = torch.empty(max(1, sdv.sd_verify_attention_workspace_size(adesc, T)), dtype=torch.uint8, device=dev)
        ws_c = torch.empty(max(1, sdv.sd_accept_reject_workspace_size(cdesc, T)), dtype=torch.uint8, device=dev)

        def attention():
            sdv.sd_verify_attention(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start,
                                    out, group_size=sp.group, max_draft=inp.max_draft, workspace=ws_a)

        def accept():
            sdv.sd_accept_reject(inp.target_logits, inp.draft_logits, inp.draft_tokens, inp.q_start,
                                 inp.uniforms, al, tok, mode=sp.mode, max_draft=inp.max_draft, workspace=ws_c)

        t_end = time.perf_counter() + max(0.0, args.settle_s)
        while time.perf_counter() < t_end:
            for _ in range(5):
                attention()
                accept()
            torch.cuda.synchronize()
        for _ in range(max(1, args.warmup)):
            attention()
            accept()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for k in range(args.steps):
            ev[k][0].record()
            attention()
            ev[k][1].record()
            accept()
            ev[k][2].record()
        torch.cuda.synchronize()
        a_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        c_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        a_bytes, a_flops = algorithmic_attention(inp)
        points.append({"D": D, "rows_per_kv_head": sp.group * (1 + D), "attention_ms": a_ms, "accept_ms": c_ms,
                       "verified_tokens_per_s": T / ((a_ms + c_ms) * 1e-3),
                       "mean_accept_len": float(al.float().mean().item()),
                       "hbm_frac": a_bytes / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "mfma_frac": a_flops / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS})
        print(f"[bench] sweep D={D}: attention {a_ms * 1e3:.1f} us, accept {c_ms * 1e3:.1f} us", file=sys.stderr,
              flush=True)
        del inp, out, ws_a, ws_c
        torch.cuda.empty_cache()
    sp = preset(SWEEP_PRESET)
    print(json.dumps({"metric": "verify attention time per draft length (tile-boundary sweep)", "unit": "ms",
                      "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": sp.name.replace("_sweep", ""), "batch": sp.batch,
                                 "kv_heads": sp.kv_heads, "group": sp.group, "head_dim": sp.head_dim,
                                 "kv_len": sp.kv_len, "vocab": sp.vocab, "alpha": alpha, "seed": args.seed},
                      "clock_settle_s_per_point": args.settle_s, "sweep": points}), flush=True)


def write_sweep_profile(sweep_json: str):
    """Text table of a --sweep line under profiles/."""
    with open(sweep_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    cfg = line["config"]
    path = os.path.join(ROOT, "profiles", f"verify_attn_sweep_{cfg['workload']}.txt")
    with open(path, "w") as f:
        f.write(f"# Verify attention per draft length D on {cfg['workload']} (one MI355X, HIP events, "
                f"{line['steps']} timed calls per point after {line['clock_settle_s_per_point']} s of clock settle).\n"
                "# G*(1+D) query rows share each KV head; the kernel variant changes at 64 rows (16x16 MFMA ->\n"
                "# 32x32 MFMA, the wave sets split the tiles), at 128 rows (rows past 128 one 16-row block of\n"
                "# 16x16 MFMAs), at 144 rows (one or two 32-row blocks past 128, split by tile parity) and at\n"
                "# 192 rows (the wave sets split the rows, so every wave takes both tiles of a step).\n"
                "$ python3 REPO/bench.py --sweep\n")
        f.write("D,rows_per_kv_head,attention_us,accept_us,hbm_frac,mfma_frac,verified_tokens_per_s,mean_AL\n")
        for pt in line["sweep"]:
            f.write(f"{pt['D']},{pt['rows_per_kv_head']},{pt['attention_ms'] * 1e3:.1f},{pt['accept_ms'] * 1e3:.1f},"
                    f"{pt['hbm_frac']:.3f},{pt['mfma_frac']:.3f},{pt['verified_tokens_per_s']:.0f},"
                    f"{pt['mean_accept_len']:.2f}\n")
    print(f"wrote {path}")


def run_linear_sweep(args):
    """The verify-shaped linear layer y = x W^T at N = K = 6144 (the expert GEMM
    of the co-design page's Figure 3) for M = batch * (1+D): TFLOP/s per batch
    and draft length, one JSON line.  W (75 MB) fits the Infinity Cache, so a
    1 GiB read evicts it before every timed call."""
    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv
    from workloads import EXPERT_K, EXPERT_N, linear_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = K = EXPERT_N
    drafts = [0, 1, 3, 7, 15]
    batches = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]
    m_max = max(b * (1 + d) for b in batches for d in drafts)
    xs, w = linear_inputs(m_max, N, K, seed=args.seed, device=dev)
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    ys = torch.empty(m_max, N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, max(sdv.sd_verify_linear_workspace_size(sdv.linear_desc(b * (1 + d), N, K))
                                for b in batches for d in drafts)), dtype=torch.uint8, device=dev)
    t_end = time.perf_counter() + max(0.0, args.settle_s)
    while time.perf_counter() < t_end:
        sdv.sd_verify_linear(xs[:512], w, ys[:512], workspace=ws)
        torch.cuda.synchronize()
    points = []
    for d in drafts:
        for b in batches:
            m = b * (1 + d)
            x, y = xs[:m], ys[:m]
            for _ in range(3):
                sdv.sd_verify_linear(x, w, y, workspace=ws)
            times = []
            for _ in range(args.steps):
                torch.amax(scratch, dim=0, keepdim=True, out=sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                sdv.sd_verify_linear(x, w, y, workspace=ws)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            t = float(np.median(times)) * 1e-3
            flops = 2.0 * m * N * K
            nbytes = 2.0 * (m * K + N * K + m * N)
            points.append({"D": d, "batch": b, "m": m, "us": t * 1e6, "tflops": flops / t / 1e12,
                           "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS,
                           "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS})
            print(f"[bench] linear D={d} batch={b} m={m}: {t * 1e6:.1f} us, {flops / t / 1e12:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
    base = next(p["tflops"] for p in points if p["D"] == 0 and p["batch"] == 1)
    for p in points:
        p["tflops_vs_D0_batch1"] = p["tflops"] / base
    print(json.dumps({"metric": "verify-shaped linear layer TFLOP/s per batch and draft length (N = K = 6144)",
                      "unit": "TFLOP/s", "higher_is_better": True, "n_gpus": 1, "steps": args.steps,
                      "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "linear_n6144_k6144", "n": N, "k": K, "drafts": drafts,
                                 "batches": batches, "seed": args.seed},
                      "cache_flush": "1 GiB scratch read before every timed call", "sweep": points}), flush=True)


def write_linear_profile(sweep_json: str):
    """Text table of a --linear-sweep line under profiles/."""
    with open(sweep_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    pts = line["sweep"]
    drafts = line["config"]["drafts"]
    batches = line["config"]["batches"]
    path = os.path.join(ROOT, "profiles", "verify_linear_sweep_n6144_k6144.txt")
    with open(path, "w") as f:
        f.write("# Verify-shaped linear layer y = x W^T, N = K = 6144, M = batch * (1+D), bf16 in / fp32 accumulate,\n"
                f"# one MI355X, median of {line['steps']} HIP-event-timed calls, each after a 1 GiB cache-evicting read.\n"
                "$ python3 REPO/bench.py --linear-sweep\n")
        f.write("TFLOP/s\nbatch," + ",".join(f"D={d}" for d in drafts) + "\n")
        for b in batches:
            f.write(f"{b}," + ",".join(f"{next(p['tflops'] for p in pts if p['D'] == d and p['batch'] == b):.1f}"
                                       for d in drafts) + "\n")
        f.write("time us\nbatch," + ",".join(f"D={d}" for d in drafts) + "\n")
        for b in batches:
            f.write(f"{b}," + ",".join(f"{next(p['us'] for p in pts if p['D'] == d and p['batch'] == b):.1f}"
                                       for d in drafts) + "\n")
    print(f"wrote {path}")


def run_probes(args):
    """On-box microbenchmarks (libsdprobe.so): the bf16 MFMA throughput of
    independent 32x32x16 and 16x16x32 chains at one and two waves per SIMD
    (HIP events for the rate, s_memtime for cycles per MFMA and the clock), and
    the SIMD each wave of an 8-wave, one-per-CU workgroup runs on.  One JSON line."""
    import ctypes
    import numpy as np
    import torch

    from speculative_decoding_verification_sd_amd.build import HERE, PROBE_LIB
    path = os.path.join(HERE, PROBE_LIB)
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build it with python -m speculative_decoding_verification_sd_amd.build")
    lib = ctypes.CDLL(path)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"cus": cus}
    # wave placement
    lay = torch.full((cus * 8,), -1, dtype=torch.int32, device=dev)
    assert lib.sdp_wave_layout(ctypes.c_void_p(lay.data_ptr()), cus, stream) == 0
    torch.cuda.synchronize()
    v = lay.cpu().numpy().reshape(cus, 8)
    simd = v & 15
    res["wave_simd_histogram"] = {f"wave{w}": {int(k): int(c) for k, c in zip(*np.unique(simd[:, w], return_counts=True))}
                                  for w in range(8)}
    res["waves_sharing_a_simd"] = sorted({tuple(int(w) for w in np.nonzero(simd[b] == s)[0])
                                          for b in range(cus) for s in range(4)})
    # MFMA peak
    iters = 20000
    for shape, chains, flops in ((32, 4, 32 * 32 * 16 * 2), (16, 8, 16 * 16 * 32 * 2)):
        for wps in (1, 2):
            grid = cus * wps
            out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
            cyc = torch.empty(grid, dtype=torch.int64, device=dev)
            args_ = (shape, grid, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(cyc.data_ptr()), stream)
            for _ in range(3):
                lib.sdp_mfma_peak(*args_)
            torch.cuda.synchronize()
            times = []
            for _ in range(max(3, args.steps)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                assert lib.sdp_mfma_peak(*args_) == 0
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e-3)
            t = float(np.median(times))
            total = grid * 4 * iters * chains * flops
            cycles = float(np.median(cyc.cpu().numpy()))
            res[f"mfma_{shape}x{shape}_{wps}wave_per_simd"] = {
                "tflops": total / t / 1e12, "frac_of_2500": total / t / 1e12 / BF16_PEAK_TFLOPS,
                "s_memtime_ticks_per_mfma_per_wave": cycles / (iters * chains),
                "us": t * 1e6}
    # MFMA / VALU co-execution: time of each variant at one and two waves per SIMD
    names = ["mfma", "mfma+2exp", "2exp", "mfma+8fma", "8fma"]
    co_iters = 20000
    for wps in (1, 2):
        grid = cus * wps
        out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
        row = {}
        for var, nm in enumerate(names):
            for _ in range(2):
                lib.sdp_coexec(var, grid, co_iters, ctypes.c_void_p(out.data_ptr()), stream)
            torch.cuda.synchronize()
            times = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                assert lib.sdp_coexec(var, grid, co_iters, ctypes.c_void_p(out.data_ptr()), stream) == 0
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3)
            row[nm] = float(np.median(times))
        res[f"coexec_us_{wps}wave_per_simd"] = row
    print(json.dumps({"metric": "on-box MFMA peak and wave placement", "probes": res}), flush=True)


def write_probe_profile(probe_json: str):
    with open(probe_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    path = os.path.join(ROOT, "profiles", "probe_mfma_peak_wave_layout.txt")
    with open(path, "w") as f:
        f.write("# On-box microbenchmarks (one MI355X): bf16 MFMA rate of independent chains from registers\n"
                "# (4 chains of 32x32x16 or 8 of 16x16x32 per wave, 20000 rounds; HIP events for the rate,\n"
                "# s_memtime cycles per wave), and the SIMD (HW_ID) each wave of an 8-wave workgroup that\n"
                "# holds a CU alone runs on.\n"
                "$ python3 REPO/bench.py --probe\n")
        for k, v in line["probes"].items():
            f.write(f"{k}: {json.dumps(v)}\n")
    print(f"wrote {path}")


def copy_calibration(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of `nbytes` (torch's elementwise copy), for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {reps} copies of {nbytes} bytes", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="g8_kv32k_D15")
    ap.add_argument("--draft", type=int, default=None, help="override D (every sequence)")
    ap.add_argument("--alpha", type=float, default=None, help="fixed acceptance rate for the synthetic drafter")
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--v-layout", choices=("dim", "key"), default="key",
                    help="V cache pages stored key-major [P,H,16,d] like K (default) or d-major [P,H,d,16]")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="before the warmup, run steps for this many seconds so the GPU clock settles")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="after the timed steps, copy BYTES device-to-device (counter calibration)")
    ap.add_argument("--sweep", nargs="*", type=int, default=None, metavar="D",
                    help="attention time per draft length on the sweep workload (default D = 0..31)")
    ap.add_argument("--write-sweep-profile", metavar="SWEEP_JSON", help="write the profiles/ table of a --sweep line")
    ap.add_argument("--linear-sweep", action="store_true",
                    help="the verify-shaped linear layer (N = K = 6144) over batch and draft length")
    ap.add_argument("--write-linear-profile", metavar="SWEEP_JSON",
                    help="write the profiles/ table of a --linear-sweep line")
    ap.add_argument("--write-profiles", nargs=4, metavar=("BENCH_JSON", "KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from a bench line and three rocprofv3 runs (no GPU)")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="verify attention time against the batch size (16 x 32K keys .. 4096 x 256 keys)")
    ap.add_argument("--write-batch-profile", nargs=2, metavar=("BENCH_JSON", "KT_DIR"),
                    help="write the profiles/ table of a --batch-sweep line and its kernel trace")
    ap.add_argument("--tree", action="store_true",
                    help="tree verification (ancestor-mask attention + greedy path acceptance), binary tree of depth 4")
    ap.add_argument("--write-tree-profile", nargs=2, metavar=("BENCH_JSON", "KT_DIR"),
                    help="write the profiles/ summary of a --tree line and its rocprofv3 kernel trace (no GPU)")
    ap.add_argument("--lossy", action="store_true",
                    help="acceptance relaxed by the Jensen-Shannon distance, beside the lossless call")
    ap.add_argument("--js-threshold", type=float, default=0.3, help="JS-distance threshold of --lossy")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="HBM read rate of a plain library reduction over 2 GiB (the practical read ceiling)")
    ap.add_argument("--loop", action="store_true",
                    help="the closed adaptive speculative-decoding loop on a bigram toy LM (graphs vs direct)")
    ap.add_argument("--write-loop-profile", nargs=2, metavar=("BENCH_JSON", "KT_DIR"),
                    help="write the profiles/ summary of a --loop line and its rocprofv3 kernel trace (no GPU)")
    ap.add_argument("--probe", action="store_true",
                    help="on-box MFMA peak and wave-to-SIMD placement microbenchmarks (libsdprobe.so)")
    ap.add_argument("--write-probe-profile", metavar="PROBE_JSON", help="write the profiles/ summary of a --probe line")
    ap.add_argument("--write-counter-profile", nargs="+", metavar="ARG",
                    help="LABEL 'BENCH_ARGS' PASS_DIR...: write the profiles/ counter summary of the attention kernel")
    ap.add_argument("--write-bench-lines", nargs="+", metavar="BENCH_JSON",
                    help="write the profiles/ table of bench lines, one per workload (no GPU)")
    ap.add_argument("--write-lossy-profile", nargs=2, metavar=("BENCH_JSON", "KT_DIR"),
                    help="write the profiles/ summary of a --lossy line and its rocprofv3 kernel trace (no GPU)")
    args = ap.parse_args()
    if args.write_probe_profile:
        write_probe_profile(args.write_probe_profile)
        return
    if args.write_counter_profile:
        write_counter_profile(*args.write_counter_profile)
        return
    if args.write_tree_profile:
        write_tree_profile(*args.write_tree_profile)
        return
    if args.write_lossy_profile:
        write_lossy_profile(*args.write_lossy_profile)
        return
    if args.write_bench_lines:
        write_bench_lines(*args.write_bench_lines)
        return
    if args.write_loop_profile:
        write_loop_profile(*args.write_loop_profile)
        return
    if args.write_profiles:
        write_profiles(*args.write_profiles, copy_bytes=args.calibrate_copy or (1 << 30))
        return
    if args.write_sweep_profile:
        write_sweep_profile(args.write_sweep_profile)
        return
    if args.write_batch_profile:
        write_batch_profile(*args.write_batch_profile)
        return
    if args.write_linear_profile:
        write_linear_profile(args.write_linear_profile)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verify step is built and timed on a single MI355X "
              "(--gpus 1); the path is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.linear_sweep:
        args.settle_s = min(args.settle_s, 0.5)
        run_linear_sweep(args)
        return
    if args.tree:
        run_tree(args)
        return
    if args.batch_sweep:
        run_batch_sweep(args)
        return
    if args.lossy:
        run_lossy(args)
        return
    if args.loop:
        run_loop(args)
        return
    if args.read_ceiling:
        run_read_ceiling(args)
        return
    if args.probe:
        run_probes(args)
        return
    if args.sweep is not None:
        args.sweep = args.sweep or list(range(32))
        if args.steps == 50 and args.warmup == 5:
            args.steps, args.warmup = 10, 3
        args.settle_s = min(args.settle_s, 0.3)
        run_sweep(args)
        return

    import numpy as np
    import torch

    import speculative_decoding_verification_sd_amd as sdv
    from workloads import generate, preset

    over = {"seed": args.seed}
    if args.draft is not None:
        over["draft_len"] = args.draft
    if args.alpha is not None:
        over["alpha"] = args.alpha
    over["v_layout"] = args.v_layout
    sp = preset(args.workload, **over)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {sp.name} on {dev}", file=sys.stderr, flush=True)
    inp = generate(sp, device=dev)
    torch.cuda.synchronize()
    B = sp.batch
    T = inp.q.shape[0]
    out = torch.empty_like(inp.q)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(T, dtype=torch.int32, device=dev)
    adesc = sdv.attn_desc(inp.q, inp.k_cache, inp.block_table, sp.group, inp.max_draft, kv_chunk=args.kv_chunk)
    cdesc = sdv.accept_desc(B, sp.vocab, inp.max_draft, sp.mode)
    ws_a = torch.empty(max(1, sdv.sd_verify_attention_workspace_size(adesc, T)), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, sdv.sd_accept_reject_workspace_size(cdesc, T)), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(1, sdv.sd_verify_step_workspace_size(adesc, cdesc, T)), dtype=torch.uint8, device=dev)

    def attention():
        sdv.sd_verify_attention(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start, out,
                                group_size=sp.group, max_draft=inp.max_draft, kv_chunk=args.kv_chunk,
                                workspace=ws_a)

    def accept():
        sdv.sd_accept_reject(inp.target_logits, inp.draft_logits, inp.draft_tokens, inp.q_start, inp.uniforms,
                             al, tok, mode=sp.mode, max_draft=inp.max_draft, workspace=ws_c)

    def step():
        sdv.sd_verify_step(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start, out,
                           inp.target_logits, inp.draft_logits, inp.draft_tokens, inp.uniforms, al, tok,
                           group_size=sp.group, max_draft=inp.max_draft, mode=sp.mode, kv_chunk=args.kv_chunk,
                           workspace=ws_s)

    # From idle the GPU takes tens of milliseconds to reach its steady clock under this load (at the
    # power limit for the attention); a few warmup steps alone would time that ramp.
    settle_steps = 0
    t_end = time.perf_counter() + max(0.0, args.settle_s)
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        settle_steps += 10
    print(f"[bench] clock settle: {settle_steps} steps in {args.settle_s:.1f} s; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    K = args.steps
    a_bytes, a_flops = algorithmic_attention(inp)
    c_bytes = algorithmic_accept(inp)
    # Between steps, outside the timed events, a 1 GiB scratch read evicts the 256 MB Infinity
    # Cache, so that no step finds the previous step's logits or pages there (the K/V stream
    # carries the non-temporal hint and need not evict them itself).  A read, not a write, so
    # that no dirty lines are left to be written back inside the timed step.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(K):
        torch.amax(scratch, dim=0, keepdim=True, out=sink)
        ev[k][0].record()
        attention()
        ev[k][1].record()
        accept()
        ev[k][2].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    attn_ms = np.asarray([ev[k][0].elapsed_time(ev[k][1]) for k in range(K)])
    acc_ms = np.asarray([ev[k][1].elapsed_time(ev[k][2]) for k in range(K)])
    step_ms = attn_ms + acc_ms
    ms_per_step = float(np.median(step_ms))
    p1090 = lambda a: [float(np.percentile(a, 10)), float(np.percentile(a, 90))]
    print(f"[bench] {K} steps: median {ms_per_step:.3f} ms/step (attention {np.median(attn_ms):.3f} ms, "
          f"accept {np.median(acc_ms):.3f} ms)", file=sys.stderr, flush=True)

    t_attn = float(np.median(attn_ms)) * 1e-3
    achieved = a_bytes / t_attn / 1e9
    mean_al = float(al.float().mean().item())

    line = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": sp.name, "batch": B, "kv_heads": sp.kv_heads, "group": sp.group, "head_dim": sp.head_dim,
            "kv_len": sp.kv_len if not isinstance(sp.kv_len, tuple) else list(sp.kv_len),
            "draft_len": sp.draft_len if not isinstance(sp.draft_len, tuple) else list(sp.draft_len),
            "vocab": sp.vocab, "accept": sp.mode, "alpha": sp.alpha, "page_size": sp.page_size,
            "verified_tokens_per_step": T, "seed": sp.seed, "v_layout": args.v_layout,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(sp.name),
            "kernel": "verify attention (plan + main + split-KV combine launches)",
            "algorithmic_bytes_per_launch": a_bytes,
            "mfma_tflops": a_flops / t_attn / 1e12, "mfma_frac": a_flops / t_attn / 1e12 / BF16_PEAK_TFLOPS,
        },
        "timing": "median of the timed steps (HIP events on the stream the calls run on); p10-p90 beside it",
        "step_ms_p10_p90": p1090(step_ms),
        "step_ms_mean": float(step_ms.mean()),
        "attention_ms": float(np.median(attn_ms)),
        "attention_ms_p10_p90": p1090(attn_ms),
        "accept_ms": float(np.median(acc_ms)),
        "accept_ms_p10_p90": p1090(acc_ms),
        "accept_gbs": c_bytes / (float(np.median(acc_ms)) * 1e-3) / 1e9,
        "accept_hbm_frac": c_bytes / (float(np.median(acc_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_accept_bytes": c_bytes,
        "step_us": ms_per_step * 1e3,
        "emitted_tokens_per_s": float(al.sum().item()) / (ms_per_step * 1e-3),
        "mean_accept_len": mean_al,
        "host_wall_s": t_wall,
        "clock_settle": {"seconds": args.settle_s, "steps": settle_steps},
        "cache_flush": "1 GiB scratch read before every timed step, outside the timed events",
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample and comparing it with the GPU outputs",
              file=sys.stderr, flush=True)
        line["cpu_baseline"], line["parity"] = cpu_baseline(inp, gpu_out=out, gpu_al=al, gpu_tok=tok)
    if args.calibrate_copy > 0:
        copy_calibration(args.calibrate_copy)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
