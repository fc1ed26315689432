"""Thin Python binding of libsdverify's C ABI (argument marshalling only).

Every function here has the name of the C entry point it calls.  Tensors are
PyTorch device tensors: PyTorch provides device memory and the stream, the
HIP library does all of the computation.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SDVERIFY_LIB") or os.path.join(HERE, "libsdverify.so")

SD_OK, SD_ERR_INVALID_ARG, SD_ERR_UNSUPPORTED, SD_ERR_WORKSPACE, SD_ERR_HIP = range(5)
SD_ACCEPT_GREEDY, SD_ACCEPT_STOCHASTIC = 0, 1
SD_OUT_BF16, SD_OUT_F32 = 0, 1
SD_V_KEY_MAJOR, SD_V_DIM_MAJOR = 0, 1
MODES = {"greedy": SD_ACCEPT_GREEDY, "stochastic": SD_ACCEPT_STOCHASTIC}


class SdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sd status {status}: {msg}")
        self.status = status


class sd_attn_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_draft", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("out_dtype", ctypes.c_int32),
        ("kv_chunk", ctypes.c_int32),
        ("v_layout", ctypes.c_int32),
    ]


class sd_accept_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("max_draft", ctypes.c_int32),
        ("mode", ctypes.c_int32),
    ]


class sd_linear_desc(ctypes.Structure):
    _fields_ = [
        ("m", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("k", ctypes.c_int32),
    ]


SD_LOOP_MAX_TIERS = 8


class sd_loop_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("ngram", ctypes.c_int32),
        ("num_tiers", ctypes.c_int32),
        ("tiers", ctypes.c_int32 * SD_LOOP_MAX_TIERS),
        ("ema_weight", ctypes.c_float),
        ("use_graphs", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I = ctypes.c_int32

SIGNATURES = {
    "sd_verify_attention_workspace_size": (_SZ, [ctypes.POINTER(sd_attn_desc), _I]),
    "sd_verify_attention": (ctypes.c_int, [ctypes.POINTER(sd_attn_desc), _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _SZ, _P]),
    "sd_accept_reject_workspace_size": (_SZ, [ctypes.POINTER(sd_accept_desc), _I]),
    "sd_accept_reject": (ctypes.c_int, [ctypes.POINTER(sd_accept_desc), _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _SZ, _P]),
    "sd_accept_reject_noalloc": (ctypes.c_int, [ctypes.POINTER(sd_accept_desc), _I, _P, _P, _P, _P, _P, _P, _P,
                                                _P]),
    "sd_accept_lossy_workspace_size": (_SZ, [ctypes.POINTER(sd_accept_desc), _I]),
    "sd_accept_lossy": (ctypes.c_int, [ctypes.POINTER(sd_accept_desc), _I, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                       _P, _P, _P, _SZ, _P]),
    "sd_verify_step_workspace_size": (_SZ, [ctypes.POINTER(sd_attn_desc), ctypes.POINTER(sd_accept_desc), _I]),
    "sd_verify_step": (ctypes.c_int, [ctypes.POINTER(sd_attn_desc), ctypes.POINTER(sd_accept_desc), _I,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sd_verify_tree_attention": (ctypes.c_int, [ctypes.POINTER(sd_attn_desc), _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                                _P, _SZ, _P]),
    "sd_tree_accept_workspace_size": (_SZ, [ctypes.POINTER(sd_accept_desc), _I]),
    "sd_tree_accept": (ctypes.c_int, [ctypes.POINTER(sd_accept_desc), _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sd_closed_loop_workspace_size": (_SZ, [ctypes.POINTER(sd_loop_desc)]),
    "sd_closed_loop": (ctypes.c_int, [ctypes.POINTER(sd_loop_desc), _P, _P, _P, _I, _P, _P, _P, _SZ, _P]),
    "sd_verify_linear_workspace_size": (_SZ, [ctypes.POINTER(sd_linear_desc)]),
    "sd_verify_linear": (ctypes.c_int, [ctypes.POINTER(sd_linear_desc), _P, _P, _P, _P, _SZ, _P]),
    "sd_validate_inputs": (ctypes.c_int, [ctypes.POINTER(sd_attn_desc), ctypes.POINTER(sd_accept_desc), _I,
                                          _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sd_last_error": (ctypes.c_char_p, []),
    "sd_version": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load libsdverify.so (after torch, so both use the same HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m speculative_decoding_verification_sd_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != SD_OK:
        raise SdError(status, lib().sd_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def v_layout_of(k_cache, v_cache) -> int:
    """The sd_v_layout of a V cache from its shape: [pages, heads, page, d] like
    K (key-major) or [pages, heads, d, page] (d-major).  head_dim is 64 or 128
    and the page 16 keys, so the two never coincide.  (No V cache: key-major;
    the workspace size does not depend on it.)"""
    if v_cache is None or tuple(v_cache.shape) == tuple(k_cache.shape):
        return SD_V_KEY_MAJOR
    return SD_V_DIM_MAJOR


def attn_desc(q, k_cache, block_table, group_size: int, max_draft: int, softmax_scale: float = 0.0,
              out_dtype=torch.bfloat16, kv_chunk: int = 0, v_cache=None) -> sd_attn_desc:
    num_pages, hkv, page, d = k_cache.shape
    return sd_attn_desc(num_seqs=block_table.shape[0], num_kv_heads=hkv, group_size=group_size, head_dim=d,
                        page_size=page, max_pages_per_seq=block_table.shape[1], num_pages=num_pages,
                        max_draft=max_draft, softmax_scale=softmax_scale,
                        out_dtype=SD_OUT_F32 if out_dtype == torch.float32 else SD_OUT_BF16,
                        kv_chunk=kv_chunk, v_layout=v_layout_of(k_cache, v_cache))


def accept_desc(num_seqs: int, vocab: int, max_draft: int, mode: str) -> sd_accept_desc:
    return sd_accept_desc(num_seqs=num_seqs, vocab=vocab, max_draft=max_draft, mode=MODES[mode])


def sd_verify_attention_workspace_size(desc: sd_attn_desc, total_q: int) -> int:
    return int(lib().sd_verify_attention_workspace_size(ctypes.byref(desc), total_q))


def sd_accept_reject_workspace_size(desc: sd_accept_desc, total_q: int) -> int:
    return int(lib().sd_accept_reject_workspace_size(ctypes.byref(desc), total_q))


def sd_accept_lossy_workspace_size(desc: sd_accept_desc, total_q: int) -> int:
    return int(lib().sd_accept_lossy_workspace_size(ctypes.byref(desc), total_q))


def sd_verify_step_workspace_size(attn: sd_attn_desc, acc: sd_accept_desc, total_q: int) -> int:
    return int(lib().sd_verify_step_workspace_size(ctypes.byref(attn), ctypes.byref(acc), total_q))


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace of {workspace.numel() * workspace.element_size()} bytes < {nbytes}")
    return workspace


def _check_attention_args(q, k_cache, v_cache, block_table, kv_len, q_start, out):
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(kv_len, "kv_len", torch.int32, dev)
    _need(q_start, "q_start", torch.int32, dev)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    _need(out, "out", out.dtype, dev)
    if k_cache.dim() != 4 or v_cache.dim() != 4 or \
            tuple(v_cache.shape) not in (tuple(k_cache.shape),
                                         (k_cache.shape[0], k_cache.shape[1], k_cache.shape[3], k_cache.shape[2])):
        raise ValueError("k_cache must be [pages, kv_heads, page_size, head_dim] and v_cache the same "
                         "(key-major) or [pages, kv_heads, head_dim, page_size] (pages stored d-major)")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [total_q, query_heads, head_dim]")
    B = block_table.shape[0]
    if kv_len.shape != (B,) or q_start.shape != (B + 1,):
        raise ValueError("kv_len must be [B] and q_start [B+1]")


def sd_verify_attention(q, k_cache, v_cache, block_table, kv_len, q_start, out, *, group_size: int,
                        max_draft: int, softmax_scale: float = 0.0, kv_chunk: int = 0,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_attention_args(q, k_cache, v_cache, block_table, kv_len, q_start, out)
    desc = attn_desc(q, k_cache, block_table, group_size, max_draft, softmax_scale, out.dtype, kv_chunk, v_cache)
    total_q = q.shape[0]
    ws = _workspace(sd_verify_attention_workspace_size(desc, total_q), q.device, workspace)
    _check(lib().sd_verify_attention(ctypes.byref(desc), total_q, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_table), _ptr(kv_len), _ptr(q_start), _ptr(out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(q.device, stream)))


def _check_accept_args(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens,
                       mode):
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32)
    _need(draft_tokens, "draft_tokens", torch.int32, dev)
    _need(q_start, "q_start", torch.int32, dev)
    _need(accept_len, "accept_len", torch.int32, dev)
    _need(out_tokens, "out_tokens", torch.int32, dev)
    if mode == "stochastic":
        _need(draft_logits, "draft_logits", torch.float32, dev)
        _need(uniforms, "uniforms", torch.float32, dev)
    B = q_start.shape[0] - 1
    T, V = target_logits.shape
    if accept_len.shape != (B,) or out_tokens.shape != (T,) or draft_tokens.shape != (T - B,):
        raise ValueError("accept_len [B], out_tokens [T_q], draft_tokens [T_q - B] expected")
    if mode == "stochastic" and (draft_logits.shape != (T - B, V) or uniforms.shape != (T,)):
        raise ValueError("draft_logits [T_q - B, V] and uniforms [T_q] expected")


def sd_accept_reject(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens, *,
                     mode: str, max_draft: int, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_accept_args(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens, mode)
    B = q_start.shape[0] - 1
    T, V = target_logits.shape
    desc = accept_desc(B, V, max_draft, mode)
    ws = _workspace(sd_accept_reject_workspace_size(desc, T), target_logits.device, workspace)
    stoch = mode == "stochastic"
    _check(lib().sd_accept_reject(ctypes.byref(desc), T, _ptr(target_logits), _ptr(draft_logits if stoch else None),
                                  _ptr(draft_tokens), _ptr(q_start), _ptr(uniforms if stoch else None),
                                  _ptr(accept_len), _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(target_logits.device, stream)))


def sd_accept_lossy(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens, *,
                    mode: str, max_draft: int, js_threshold: float, draft_entropy: Optional[torch.Tensor] = None,
                    js_distance: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """Accept/reject where a draft also passes when the Jensen-Shannon distance
    of its target and draft rows is at most js_threshold (negative: lossless);
    optionally writes every drafted row's draft entropy and JS distance."""
    stoch = mode == "stochastic"
    _check_accept_args(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens, mode)
    B = q_start.shape[0] - 1
    T, V = target_logits.shape
    _need(draft_logits, "draft_logits", torch.float32, target_logits.device)
    if draft_logits.shape != (T - B, V):
        raise ValueError("draft_logits [T_q - B, V] expected")
    for t, name in ((draft_entropy, "draft_entropy"), (js_distance, "js_distance")):
        if t is not None:
            _need(t, name, torch.float32, target_logits.device)
            if t.shape != (T - B,):
                raise ValueError(f"{name} [T_q - B] expected")
    desc = accept_desc(B, V, max_draft, mode)
    ws = _workspace(sd_accept_lossy_workspace_size(desc, T), target_logits.device, workspace)
    _check(lib().sd_accept_lossy(ctypes.byref(desc), T, _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
                                 _ptr(q_start), _ptr(uniforms if stoch else None), float(js_threshold),
                                 _ptr(accept_len), _ptr(out_tokens), _ptr(draft_entropy), _ptr(js_distance),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(target_logits.device, stream)))


def loop_desc(num_seqs: int, vocab: int, max_len: int, tiers=(1, 3, 7), ngram: int = 3, ema_weight: float = 0.5,
              use_graphs: bool = True) -> sd_loop_desc:
    tiers = list(tiers)
    if not 1 <= len(tiers) <= SD_LOOP_MAX_TIERS:
        raise ValueError(f"1..{SD_LOOP_MAX_TIERS} tiers expected")
    arr = (ctypes.c_int32 * SD_LOOP_MAX_TIERS)(*(tiers + [0] * (SD_LOOP_MAX_TIERS - len(tiers))))
    return sd_loop_desc(num_seqs=num_seqs, vocab=vocab, max_len=max_len, ngram=ngram, num_tiers=len(tiers),
                        tiers=arr, ema_weight=ema_weight, use_graphs=int(bool(use_graphs)))


def sd_closed_loop_workspace_size(desc: sd_loop_desc) -> int:
    return int(lib().sd_closed_loop_workspace_size(ctypes.byref(desc)))


def sd_closed_loop(bigram_logits, history, length, *, steps: int, tiers=(1, 3, 7), ngram: int = 3,
                   ema_weight: float = 0.5, use_graphs: bool = True, workspace: Optional[torch.Tensor] = None,
                   stream=None):
    """Run `steps` rounds of the closed speculative-decoding loop on the bigram
    toy LM (bigram_logits fp32 [V, V]); history int32 [B, max_len] and length
    int32 [B] are updated in place.  Returns (accept_trace int32 [steps, B],
    tier_trace int32 [steps]) as host tensors."""
    dev = bigram_logits.device
    _need(bigram_logits, "bigram_logits", torch.float32)
    _need(history, "history", torch.int32, dev)
    _need(length, "length", torch.int32, dev)
    V = bigram_logits.shape[0]
    if bigram_logits.shape != (V, V) or history.dim() != 2 or length.shape != (history.shape[0],):
        raise ValueError("bigram_logits [V, V], history [B, max_len] and length [B] expected")
    B, max_len = history.shape
    desc = loop_desc(B, V, max_len, tiers, ngram, ema_weight, use_graphs)
    ws = _workspace(sd_closed_loop_workspace_size(desc), dev, workspace)
    pin = torch.cuda.is_available()
    al = torch.zeros((max(steps, 0), B), dtype=torch.int32, pin_memory=pin)
    tr = torch.zeros(max(steps, 0), dtype=torch.int32, pin_memory=pin)
    _check(lib().sd_closed_loop(ctypes.byref(desc), _ptr(bigram_logits), _ptr(history), _ptr(length), steps,
                                ctypes.c_void_p(al.data_ptr()), ctypes.c_void_p(tr.data_ptr()), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(dev, stream)))
    return al, tr


def sd_verify_step(q, k_cache, v_cache, block_table, kv_len, q_start, attn_out, target_logits, draft_logits,
                   draft_tokens, uniforms, accept_len, out_tokens, *, group_size: int, max_draft: int, mode: str,
                   softmax_scale: float = 0.0, kv_chunk: int = 0, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    _check_attention_args(q, k_cache, v_cache, block_table, kv_len, q_start, attn_out)
    _check_accept_args(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens, mode)
    adesc = attn_desc(q, k_cache, block_table, group_size, max_draft, softmax_scale, attn_out.dtype, kv_chunk,
                      v_cache)
    B = q_start.shape[0] - 1
    T, V = target_logits.shape
    cdesc = accept_desc(B, V, max_draft, mode)
    ws = _workspace(sd_verify_step_workspace_size(adesc, cdesc, T), q.device, workspace)
    stoch = mode == "stochastic"
    _check(lib().sd_verify_step(ctypes.byref(adesc), ctypes.byref(cdesc), T, _ptr(q), _ptr(k_cache),
                                _ptr(v_cache), _ptr(block_table), _ptr(kv_len), _ptr(q_start), _ptr(attn_out),
                                _ptr(target_logits), _ptr(draft_logits if stoch else None), _ptr(draft_tokens),
                                _ptr(uniforms if stoch else None), _ptr(accept_len), _ptr(out_tokens), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(q.device, stream)))


def sd_verify_tree_attention(q, k_cache, v_cache, block_table, kv_len, q_start, parents, out, *, group_size: int,
                             max_draft: int, softmax_scale: float = 0.0, kv_chunk: int = 0,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Verify attention under the ancestor masks of per-sequence draft trees
    (parents int32 [total_q - B]: parent of node i of sequence b at (q_start[b]-b)+i-1)."""
    _check_attention_args(q, k_cache, v_cache, block_table, kv_len, q_start, out)
    B = block_table.shape[0]
    _need(parents, "parents", torch.int32, q.device)
    if parents.shape != (q.shape[0] - B,):
        raise ValueError("parents must be [total_q - B]")
    desc = attn_desc(q, k_cache, block_table, group_size, max_draft, softmax_scale, out.dtype, kv_chunk, v_cache)
    total_q = q.shape[0]
    ws = _workspace(sd_verify_attention_workspace_size(desc, total_q), q.device, workspace)
    _check(lib().sd_verify_tree_attention(ctypes.byref(desc), total_q, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(block_table), _ptr(kv_len), _ptr(q_start), _ptr(parents), _ptr(out),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device, stream)))


def sd_tree_accept_workspace_size(desc: sd_accept_desc, total_q: int) -> int:
    return int(lib().sd_tree_accept_workspace_size(ctypes.byref(desc), total_q))


def sd_tree_accept(target_logits, tree_tokens, q_start, parents, accept_len, out_tokens, out_nodes, *,
                   max_draft: int, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Greedy acceptance of per-sequence draft trees (see the C header)."""
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32)
    for t, name in ((tree_tokens, "tree_tokens"), (q_start, "q_start"), (parents, "parents"),
                    (accept_len, "accept_len"), (out_tokens, "out_tokens"), (out_nodes, "out_nodes")):
        _need(t, name, torch.int32, dev)
    B = q_start.shape[0] - 1
    T, V = target_logits.shape
    if tree_tokens.shape != (T - B,) or parents.shape != (T - B,) or accept_len.shape != (B,) or \
            out_tokens.shape != (T,) or out_nodes.shape != (T,):
        raise ValueError("tree_tokens, parents [T_q - B]; accept_len [B]; out_tokens, out_nodes [T_q] expected")
    desc = accept_desc(B, V, max_draft, "greedy")
    ws = _workspace(sd_tree_accept_workspace_size(desc, T), dev, workspace)
    _check(lib().sd_tree_accept(ctypes.byref(desc), T, _ptr(target_logits), _ptr(tree_tokens), _ptr(q_start),
                                _ptr(parents), _ptr(accept_len), _ptr(out_tokens), _ptr(out_nodes), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(dev, stream)))


def linear_desc(m: int, n: int, k: int) -> sd_linear_desc:
    return sd_linear_desc(int(m), int(n), int(k))


def sd_verify_linear_workspace_size(desc: sd_linear_desc) -> int:
    return int(lib().sd_verify_linear_workspace_size(ctypes.byref(desc)))


def sd_verify_linear(x, w, y, *, workspace=None, stream=None):
    """y = x w^T for bf16 x [m, k], w [n, k] into bf16 y [m, n]."""
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16, x.device)
    _need(y, "y", torch.bfloat16, x.device)
    if x.dim() != 2 or w.dim() != 2 or y.dim() != 2:
        raise ValueError("x, w and y must be 2-d")
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k or tuple(y.shape) != (m, n):
        raise ValueError(f"shapes x {tuple(x.shape)}, w {tuple(w.shape)}, y {tuple(y.shape)} do not match")
    desc = linear_desc(m, n, k)
    need = sd_verify_linear_workspace_size(desc)
    ws = _workspace(need, x.device, workspace)
    _check(lib().sd_verify_linear(ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(y), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(x.device, stream)))


def sd_version() -> str:
    return lib().sd_version().decode()


def sd_last_error() -> str:
    return lib().sd_last_error().decode()


# Bits of the word sd_validate_inputs writes (0: no violation found).
SD_BAD = {"q_start": 1, "kv_len": 2, "page": 4, "token": 8, "uniform": 16, "logits": 32}


def sd_validate_inputs(q_start, *, max_draft: int, q=None, k_cache=None, block_table=None, kv_len=None,
                       group_size: int = 1, draft_tokens=None, uniforms=None, target_logits=None, draft_logits=None,
                       vocab: Optional[int] = None, status_word: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Opt-in device-side check of the inputs' contract (the verify calls only
    clamp what they index).  The attention half is checked when block_table is
    given (with q, k_cache and kv_len), the accept half when draft_tokens or
    target_logits is given; logits are scanned only when passed.  Returns the
    status word (int32 [1] on the device, stream-ordered): the OR of the
    SD_BAD bits found, 0 when the inputs keep the contract."""
    B = q_start.shape[0] - 1
    dev = q_start.device
    _need(q_start, "q_start", torch.int32, dev)
    T = next((t.shape[0] for t in (q, target_logits, uniforms) if t is not None), None)
    if T is None:
        raise ValueError("total_q comes from q, target_logits or uniforms: pass one of them")
    ad = cd = None
    if block_table is not None:
        if q is None or k_cache is None or kv_len is None:
            raise ValueError("the attention half needs q, k_cache, block_table and kv_len")
        _need(block_table, "block_table", torch.int32, dev)
        _need(kv_len, "kv_len", torch.int32, dev)
        ad = attn_desc(q, k_cache, block_table, group_size, max_draft)
    if draft_tokens is not None or target_logits is not None:
        V = target_logits.shape[1] if target_logits is not None else vocab
        if V is None:
            raise ValueError("the accept half needs target_logits or vocab")
        for t, name, dt in ((draft_tokens, "draft_tokens", torch.int32), (uniforms, "uniforms", torch.float32),
                            (target_logits, "target_logits", torch.float32),
                            (draft_logits, "draft_logits", torch.float32)):
            if t is not None:
                _need(t, name, dt, dev)
        cd = accept_desc(B, V, max_draft, "stochastic" if uniforms is not None else "greedy")
    if status_word is None:
        status_word = torch.empty(1, dtype=torch.int32, device=dev)
    _need(status_word, "status_word", torch.int32, dev)
    _check(lib().sd_validate_inputs(ctypes.byref(ad) if ad is not None else None,
                                    ctypes.byref(cd) if cd is not None else None, T,
                                    _ptr(block_table), _ptr(kv_len), _ptr(q_start), _ptr(draft_tokens),
                                    _ptr(uniforms), _ptr(target_logits), _ptr(draft_logits), _ptr(status_word),
                                    _stream(dev, stream)))
    return status_word


def sd_accept_reject_noalloc(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens,
                             *, mode: str, max_draft: int, stream=None) -> None:
    """sd_accept_reject on the library's own scratch: no workspace, nothing allocated."""
    _check_accept_args(target_logits, draft_logits, draft_tokens, q_start, uniforms, accept_len, out_tokens, mode)
    B = q_start.shape[0] - 1
    T, V = target_logits.shape
    desc = accept_desc(B, V, max_draft, mode)
    stoch = mode == "stochastic"
    _check(lib().sd_accept_reject_noalloc(ctypes.byref(desc), T, _ptr(target_logits),
                                          _ptr(draft_logits if stoch else None), _ptr(draft_tokens), _ptr(q_start),
                                          _ptr(uniforms if stoch else None), _ptr(accept_len), _ptr(out_tokens),
                                          _stream(target_logits.device, stream)))
