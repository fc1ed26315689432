"""Helpers for the GPU parity tests: run the HIP path through the binding and
compare with the oracle on the same generated inputs."""

import contextlib
import os
import sys

import numpy as np
import torch

import speculative_decoding_verification_sd_amd as sdv
from oracle import accept_greedy, accept_stochastic, verify_attention
from tests.oracle_io import accept_args, attention_args

ATTN_TOL = 2e-2   # absolute, bf16 attention outputs against the fp64 oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def on_gpu(inp):
    return inp if inp.q.is_cuda else inp.to("cuda")


def gpu_attention(inp, out_dtype=torch.bfloat16, kv_chunk=0, softmax_scale=0.0):
    x = on_gpu(inp)
    out = torch.full(x.q.shape, float("nan"), dtype=out_dtype, device=x.q.device)
    sdv.sd_verify_attention(x.q, x.k_cache, x.v_cache, x.block_table, x.kv_len, x.q_start, out,
                            group_size=inp.group, max_draft=inp.max_draft, softmax_scale=softmax_scale,
                            kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    return out


def gpu_accept(inp, mode=None):
    x = on_gpu(inp)
    mode = mode or inp.spec.mode
    B = x.q_start.shape[0] - 1
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((x.target_logits.shape[0],), -7, dtype=torch.int32, device="cuda")
    sdv.sd_accept_reject(x.target_logits, x.draft_logits, x.draft_tokens, x.q_start, x.uniforms, al, out,
                         mode=mode, max_draft=inp.max_draft)
    torch.cuda.synchronize()
    return al.cpu().numpy(), out.cpu().numpy()


def oracle_accept(inp, mode=None, margins=None):
    mode = mode or inp.spec.mode
    a = accept_args(inp)
    if mode == "greedy":
        return accept_greedy(a["target_logits"], a["draft_tokens"], a["q_start"])
    return accept_stochastic(**a, margins=margins)


def oracle_workers():
    """Threads for the oracle's independent units: the CPUs this process may
    use, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare_attention(inp, out, units=None, workers=None, tol=ATTN_TOL):
    """Max |gpu - oracle| over all rows (or over the listed (b, h) units)."""
    workers = workers or oracle_workers()
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)     # one BLAS thread per oracle thread
    except ImportError:
        ctx = contextlib.nullcontext()
    with ctx:
        ref = verify_attention(**attention_args(inp), units=units, workers=workers)
    got = out.float().cpu().numpy().astype(np.float64)
    mask = ~np.isnan(ref)
    assert np.all(np.isfinite(got[mask])), "GPU output has non-finite values where the oracle has numbers"
    err = np.abs(got[mask] - ref[mask])
    return float(err.max()) if err.size else 0.0
