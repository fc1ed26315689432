"""sd_verify_step (attention then accept on one stream, one workspace) gives
exactly what the two separate calls give, and both match the oracle."""

import numpy as np
import pytest
import torch

import speculative_decoding_verification_sd_amd as sdv
from tests.gpu_util import ATTN_TOL, compare_attention, gpu_accept, gpu_attention, oracle_accept, say
from workloads import generate, preset

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", dict(mode="greedy")),
                                       ("ragged_b64", dict(batch=6, kv_len=[5000, 70, 900, 16, 3000, 129]))])
def test_step_equals_separate_calls(name, over):
    sp = preset(name, **over)
    say(f"case: step {sp.name} {sp.mode}")
    inp = generate(sp).to("cuda")
    B = inp.q_start.shape[0] - 1
    T = inp.q.shape[0]
    out = torch.empty_like(inp.q)
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    sdv.sd_verify_step(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.kv_len, inp.q_start, out,
                       inp.target_logits, inp.draft_logits, inp.draft_tokens, inp.uniforms, al, tok,
                       group_size=sp.group, max_draft=inp.max_draft, mode=sp.mode)
    torch.cuda.synchronize()
    ref_out = gpu_attention(inp)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    al2, tok2 = gpu_accept(inp)
    assert np.array_equal(al.cpu().numpy(), al2) and np.array_equal(tok.cpu().numpy(), tok2)
    al_o, tok_o = oracle_accept(inp.to("cpu"))
    assert np.array_equal(al_o, al2) and np.array_equal(tok_o, tok2)
    assert compare_attention(inp.to("cpu"), out) <= ATTN_TOL
