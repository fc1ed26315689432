"""The C ABI library loads, exports every function include/sd_verify.h
declares, and rejects invalid host-side arguments before touching a GPU."""

import ctypes
import os
import re

import pytest

import speculative_decoding_verification_sd_amd as sdv
from speculative_decoding_verification_sd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd_verify.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls_and_their_workspace_queries():
    names = declared_functions()
    for n in ("sd_verify_attention", "sd_accept_reject", "sd_verify_step", "sd_verify_attention_workspace_size",
              "sd_accept_reject_workspace_size", "sd_verify_step_workspace_size", "sd_last_error", "sd_version"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = sdv.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in B.SIGNATURES, n
    assert sdv.sd_version().startswith("sdverify")


def _attn(**kw):
    d = dict(num_seqs=2, num_kv_heads=2, group_size=4, head_dim=64, page_size=16, max_pages_per_seq=16,
             num_pages=40, max_draft=3, softmax_scale=0.0, out_dtype=0, kv_chunk=0, v_layout=0)
    d.update(kw)
    return B.sd_attn_desc(**d)


def _acc(**kw):
    d = dict(num_seqs=2, vocab=1000, max_draft=3, mode=1)
    d.update(kw)
    return B.sd_accept_desc(**d)


def test_workspace_queries():
    assert sdv.sd_verify_attention_workspace_size(_attn(), 8) > 0
    assert sdv.sd_accept_reject_workspace_size(_acc(), 8) > 0
    assert sdv.sd_verify_step_workspace_size(_attn(), _acc(), 8) >= \
        sdv.sd_verify_attention_workspace_size(_attn(), 8) + sdv.sd_accept_reject_workspace_size(_acc(), 8)
    # invalid descriptions report 0
    assert sdv.sd_verify_attention_workspace_size(_attn(head_dim=96), 8) == 0
    assert sdv.sd_verify_attention_workspace_size(_attn(group_size=8, max_draft=32), 8) == 0
    assert sdv.sd_accept_reject_workspace_size(_acc(vocab=0), 8) == 0
    assert sdv.sd_verify_step_workspace_size(_attn(num_seqs=3), _acc(), 8) == 0
    # the largest supported rows per KV head is 256 = G*(1+D)
    assert sdv.sd_verify_attention_workspace_size(_attn(group_size=8, max_draft=31, num_seqs=1), 32) > 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(head_dim=80), B.SD_ERR_UNSUPPORTED, "head_dim"),
    (dict(page_size=32), B.SD_ERR_UNSUPPORTED, "page_size"),
    (dict(group_size=0), B.SD_ERR_INVALID_ARG, "group_size"),
    (dict(num_kv_heads=0), B.SD_ERR_INVALID_ARG, "num_kv_heads"),
    (dict(group_size=16, max_draft=16), B.SD_ERR_UNSUPPORTED, "exceeds 256"),
    (dict(kv_chunk=100), B.SD_ERR_INVALID_ARG, "kv_chunk"),
    (dict(softmax_scale=float("nan")), B.SD_ERR_INVALID_ARG, "softmax_scale"),
    (dict(out_dtype=7), B.SD_ERR_INVALID_ARG, "out_dtype"),
    (dict(v_layout=2), B.SD_ERR_INVALID_ARG, "v_layout"),
])
def test_attention_rejects_bad_descriptions(kw, status, needle):
    lib = sdv.lib()
    d = _attn(**kw)
    st = lib.sd_verify_attention(ctypes.byref(d), 8, *([None] * 8), 0, None)
    assert st == status
    assert needle in sdv.sd_last_error()


def test_attention_rejects_null_pointers_and_small_workspace():
    lib = sdv.lib()
    d = _attn()
    dummy = ctypes.c_void_p(4096)
    st = lib.sd_verify_attention(ctypes.byref(d), 8, None, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "NULL" in sdv.sd_last_error()
    st = lib.sd_verify_attention(ctypes.byref(d), 8, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 16,
                                 None)
    assert st == B.SD_ERR_WORKSPACE
    st = lib.sd_verify_attention(ctypes.byref(d), 100, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "total_q" in sdv.sd_last_error()
    st = lib.sd_verify_attention(None, 8, *([None] * 8), 0, None)
    assert st == B.SD_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op():
    lib = sdv.lib()
    d = _attn(num_seqs=0)
    assert lib.sd_verify_attention(ctypes.byref(d), 0, *([None] * 8), 0, None) == B.SD_OK
    a = _acc(num_seqs=0)
    assert lib.sd_accept_reject(ctypes.byref(a), 0, *([None] * 8), 0, None) == B.SD_OK


def test_accept_rejects_bad_arguments():
    lib = sdv.lib()
    dummy = ctypes.c_void_p(4096)
    a = _acc(mode=5)
    assert lib.sd_accept_reject(ctypes.byref(a), 8, *([dummy] * 8), 1 << 30, None) == B.SD_ERR_INVALID_ARG
    a = _acc()
    # stochastic without uniforms
    st = lib.sd_accept_reject(ctypes.byref(a), 8, dummy, dummy, dummy, dummy, None, dummy, dummy, dummy, 1 << 30,
                              None)
    assert st == B.SD_ERR_INVALID_ARG and "uniforms" in sdv.sd_last_error()
    st = lib.sd_accept_reject(ctypes.byref(a), 8, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 8, None)
    assert st == B.SD_ERR_WORKSPACE
    a = _acc(mode=0)
    # greedy may omit draft logits and uniforms, but not the workspace
    st = lib.sd_accept_reject(ctypes.byref(a), 8, dummy, None, dummy, dummy, None, dummy, dummy, None, 0, None)
    assert st == B.SD_ERR_WORKSPACE


def test_step_checks_consistency():
    lib = sdv.lib()
    d = _attn()
    a = _acc(num_seqs=3)
    st = lib.sd_verify_step(ctypes.byref(d), ctypes.byref(a), 8, *([None] * 14), 0, None)
    assert st == B.SD_ERR_INVALID_ARG and "num_seqs" in sdv.sd_last_error()


def test_binding_validates_tensors_on_cpu():
    import torch
    q = torch.zeros(8, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        sdv.sd_verify_attention(q, q, q, torch.zeros(2, 16, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                                torch.zeros(3, dtype=torch.int32), q, group_size=4, max_draft=3)


def test_linear_workspace_and_rejections():
    lib = sdv.lib()
    # small m splits K (fp32 partials in the workspace); a large m needs none
    assert sdv.sd_verify_linear_workspace_size(sdv.linear_desc(8, 6144, 6144)) > 0
    assert sdv.sd_verify_linear_workspace_size(sdv.linear_desc(4096, 6144, 6144)) == 0
    for (m, n, k), status, needle in [((8, 100, 64), B.SD_ERR_UNSUPPORTED, "n="),
                                      ((8, 128, 100), B.SD_ERR_UNSUPPORTED, "k="),
                                      ((-1, 128, 64), B.SD_ERR_INVALID_ARG, "m="),
                                      ((8, 0, 64), B.SD_ERR_INVALID_ARG, "n=")]:
        d = sdv.linear_desc(m, n, k)
        assert sdv.sd_verify_linear_workspace_size(d) == 0
        assert lib.sd_verify_linear(ctypes.byref(d), None, None, None, None, 0, None) == status
        assert needle in sdv.sd_last_error()
    dummy = ctypes.c_void_p(4096)
    d = sdv.linear_desc(8, 6144, 6144)
    assert lib.sd_verify_linear(ctypes.byref(d), None, dummy, dummy, dummy, 1 << 30, None) == B.SD_ERR_INVALID_ARG
    assert lib.sd_verify_linear(ctypes.byref(d), dummy, dummy, dummy, dummy, 16, None) == B.SD_ERR_WORKSPACE
    assert lib.sd_verify_linear(ctypes.byref(d), ctypes.c_void_p(4100), dummy, dummy, dummy, 1 << 30,
                                None) == B.SD_ERR_INVALID_ARG
    assert lib.sd_verify_linear(None, None, None, None, None, 0, None) == B.SD_ERR_INVALID_ARG
    # m = 0 is a no-op
    d = sdv.linear_desc(0, 128, 64)
    assert lib.sd_verify_linear(ctypes.byref(d), None, None, None, None, 0, None) == B.SD_OK


def test_tree_calls_reject_bad_arguments():
    lib = sdv.lib()
    dummy = ctypes.c_void_p(4096)
    # trees are greedy only and hold at most 64 nodes
    a = _acc(mode=1)
    assert sdv.sd_tree_accept_workspace_size(a, 8) == 0
    st = lib.sd_tree_accept(ctypes.byref(a), 8, *([dummy] * 7), dummy, 1 << 30, None)
    assert st == B.SD_ERR_UNSUPPORTED and "greedily" in sdv.sd_last_error()
    a = _acc(mode=0, max_draft=64)
    assert sdv.sd_tree_accept_workspace_size(a, 8) == 0
    st = lib.sd_tree_accept(ctypes.byref(a), 8, *([dummy] * 7), dummy, 1 << 30, None)
    assert st == B.SD_ERR_UNSUPPORTED and "64 nodes" in sdv.sd_last_error()
    a = _acc(mode=0)
    assert sdv.sd_tree_accept_workspace_size(a, 8) > 0
    st = lib.sd_tree_accept(ctypes.byref(a), 8, dummy, dummy, dummy, None, dummy, dummy, dummy, dummy, 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "NULL" in sdv.sd_last_error()
    st = lib.sd_tree_accept(ctypes.byref(a), 8, *([dummy] * 7), dummy, 8, None)
    assert st == B.SD_ERR_WORKSPACE
    d = _attn(max_draft=64, group_size=1)
    st = lib.sd_verify_tree_attention(ctypes.byref(d), 8, *([dummy] * 8), dummy, 1 << 30, None)
    assert st == B.SD_ERR_UNSUPPORTED and "64 nodes" in sdv.sd_last_error()
    d = _attn()
    st = lib.sd_verify_tree_attention(ctypes.byref(d), 8, *([dummy] * 6), None, dummy, dummy, 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "parents" in sdv.sd_last_error()


def test_lossy_call_rejects_bad_arguments():
    lib = sdv.lib()
    dummy = ctypes.c_void_p(4096)
    a = _acc(mode=0)
    assert sdv.sd_accept_lossy_workspace_size(a, 8) > sdv.sd_accept_reject_workspace_size(a, 8)
    # greedy still needs the draft logits (the JS distance compares both distributions)
    st = lib.sd_accept_lossy(ctypes.byref(a), 8, dummy, None, dummy, dummy, None, ctypes.c_float(0.1), dummy,
                             dummy, None, None, dummy, 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "draft_logits" in sdv.sd_last_error()
    st = lib.sd_accept_lossy(ctypes.byref(a), 8, dummy, dummy, dummy, dummy, None, ctypes.c_float(float("nan")),
                             dummy, dummy, None, None, dummy, 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "NaN" in sdv.sd_last_error()
    st = lib.sd_accept_lossy(ctypes.byref(a), 8, dummy, dummy, dummy, dummy, None, ctypes.c_float(0.1),
                             dummy, dummy, None, None, dummy, 8, None)
    assert st == B.SD_ERR_WORKSPACE
    a = _acc(mode=1)
    st = lib.sd_accept_lossy(ctypes.byref(a), 8, dummy, dummy, dummy, dummy, None, ctypes.c_float(0.1),
                             dummy, dummy, None, None, dummy, 1 << 30, None)
    assert st == B.SD_ERR_INVALID_ARG and "uniforms" in sdv.sd_last_error()


def test_closed_loop_rejects_bad_descriptions():
    lib = sdv.lib()
    dummy = ctypes.c_void_p(4096)
    ok = sdv.loop_desc(4, 100, 64)
    assert sdv.sd_closed_loop_workspace_size(ok) > 0
    for kw, status, needle in [(dict(tiers=(3, 1)), B.SD_ERR_INVALID_ARG, "ascending"),
                               (dict(tiers=(1, 64)), B.SD_ERR_UNSUPPORTED, "tier"),
                               (dict(ngram=9), B.SD_ERR_UNSUPPORTED, "ngram"),
                               (dict(ema_weight=0.0), B.SD_ERR_INVALID_ARG, "ema_weight"),
                               (dict(max_len=1), B.SD_ERR_INVALID_ARG, "max_len")]:
        args = dict(num_seqs=4, vocab=100, max_len=64)
        args.update(kw)
        d = sdv.loop_desc(**args)
        assert sdv.sd_closed_loop_workspace_size(d) == 0
        assert lib.sd_closed_loop(ctypes.byref(d), dummy, dummy, dummy, 3, dummy, dummy, dummy, 1 << 30,
                                  None) == status
        assert needle in sdv.sd_last_error()
    assert lib.sd_closed_loop(ctypes.byref(ok), dummy, dummy, dummy, 3, None, dummy, dummy, 1 << 30,
                              None) == B.SD_ERR_INVALID_ARG
    assert lib.sd_closed_loop(ctypes.byref(ok), dummy, dummy, dummy, 3, dummy, dummy, dummy, 8,
                              None) == B.SD_ERR_WORKSPACE
    assert lib.sd_closed_loop(ctypes.byref(ok), None, None, None, 0, None, None, None, 0, None) == B.SD_OK


_FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails before anything is enqueued


@pytest.mark.parametrize("case,needle", [
    ("no_desc", "needs an attention or an accept descriptor"),
    ("disagree", "disagree on num_seqs or max_draft"),
    ("no_status", "status_word and q_start are required"),
    ("no_table", "block_table and kv_len are required"),
    ("no_tokens", "draft_tokens is required"),
    ("bad_attn", "head_dim"),
])
def test_validate_inputs_rejects_bad_arguments(case, needle):
    lib = sdv.lib()
    a, c = _attn(), _acc()
    args = dict(attn=ctypes.byref(a), acc=ctypes.byref(c), table=_FAKE, kv=_FAKE, qs=_FAKE, tok=_FAKE, status=_FAKE)
    if case == "no_desc":
        args.update(attn=None, acc=None)
    elif case == "disagree":
        c2 = _acc(max_draft=5)
        args.update(acc=ctypes.byref(c2))
    elif case == "no_status":
        args.update(status=None)
    elif case == "no_table":
        args.update(table=None)
    elif case == "no_tokens":
        args.update(tok=None)
    elif case == "bad_attn":
        a2 = _attn(head_dim=96)
        args.update(attn=ctypes.byref(a2))
    st = lib.sd_validate_inputs(args["attn"], args["acc"], 8, args["table"], args["kv"], args["qs"], args["tok"],
                                None, None, None, args["status"], None)
    assert st != B.SD_OK
    assert needle in sdv.sd_last_error()


def test_v_layout_from_the_cache_shape():
    """The binding passes the V cache's page layout from its shape: [P, H, 16, d]
    like K is key-major, [P, H, d, 16] d-major; any other shape is refused."""
    import torch
    k = torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16)
    assert B.v_layout_of(k, torch.zeros(4, 2, 16, 64)) == B.SD_V_KEY_MAJOR
    assert B.v_layout_of(k, torch.zeros(4, 2, 64, 16)) == B.SD_V_DIM_MAJOR
