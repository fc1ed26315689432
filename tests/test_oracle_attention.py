"""Pins of the attention oracle against things other than itself.

* a library routine: torch's scaled_dot_product_attention in fp64 on dense
  per-sequence K/V with the lower-right causal mask (queries are the last rows
  of the sequence) and K/V repeated per query head;
* invariants: row i of a verify block equals plain decode attention over the
  first N-D+i keys; relabelling physical pages changes nothing;
* closed forms: constant V gives V; a single dominant key gives its V; a
  vanishing scale gives the mean of the visible V rows.
"""

import math

import numpy as np
import pytest
import torch
from torch.nn.attention.bias import causal_lower_right

from oracle import verify_attention, verify_attention_unit, bf16_bits_to_f64


def _paged_from_dense(dense_k, dense_v, page, rng, extra_pages=3):
    """Scatter dense per-sequence K/V (list of [Hkv, N_b, d] bf16 bit arrays) into a
    randomly permuted page pool; returns (k_bits, v_bits, block_table)."""
    B = len(dense_k)
    Hkv, _, d = dense_k[0].shape
    npages = [(k.shape[1] + page - 1) // page for k in dense_k]
    pool = sum(npages) + extra_pages
    perm = rng.permutation(pool)
    kc = rng.integers(0, 1 << 16, size=(pool, Hkv, page, d), dtype=np.uint16)   # junk everywhere
    vc = rng.integers(0, 1 << 16, size=(pool, Hkv, d, page), dtype=np.uint16)   # pages stored d-major
    # keep junk finite so that it cannot hide behind NaN arithmetic
    kc &= np.uint16(0x3FFF)
    vc &= np.uint16(0x3FFF)
    bt = np.full((B, max(npages)), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        for pg in range(npages[b]):
            phys = perm[off]
            off += 1
            bt[b, pg] = phys
            lo, hi = pg * page, min((pg + 1) * page, dense_k[b].shape[1])
            kc[phys, :, : hi - lo, :] = dense_k[b][:, lo:hi, :]
            vc[phys, :, :, : hi - lo] = dense_v[b][:, lo:hi, :].transpose(0, 2, 1)
    return kc, vc, bt


def _rand_bits(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def _case(rng, lens, drafts, Hkv, G, d, page=16):
    dk = [_rand_bits(rng, (Hkv, n, d)) for n in lens]
    dv = [_rand_bits(rng, (Hkv, n, d)) for n in lens]
    kc, vc, bt = _paged_from_dense(dk, dv, page, rng)
    q_start = np.concatenate([[0], np.cumsum(np.asarray(drafts) + 1)]).astype(np.int32)
    q = _rand_bits(rng, (int(q_start[-1]), Hkv * G, d))
    return dict(q=q, kc=kc, vc=vc, bt=bt, kv_len=np.asarray(lens, dtype=np.int32), q_start=q_start,
                dense_k=dk, dense_v=dv, G=G)


@pytest.mark.parametrize("G,d,lens,drafts", [
    (4, 64, [40, 17], [3, 0]),
    (2, 32, [16, 33, 5], [2, 4, 1]),
    (8, 16, [64], [7]),
])
def test_matches_sdpa_lower_right_causal(G, d, lens, drafts):
    rng = np.random.default_rng(11)
    c = _case(rng, lens, drafts, Hkv=3, G=G, d=d)
    out = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], G)
    for b, n in enumerate(lens):
        t0, t1 = c["q_start"][b], c["q_start"][b + 1]
        L = t1 - t0
        qd = torch.from_numpy(bf16_bits_to_f64(c["q"][t0:t1])).permute(1, 0, 2)          # [Hq, L, d]
        kd = torch.from_numpy(bf16_bits_to_f64(c["dense_k"][b])).repeat_interleave(G, 0)  # [Hq, N, d]
        vd = torch.from_numpy(bf16_bits_to_f64(c["dense_v"][b])).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qd[None], kd[None], vd[None], attn_mask=causal_lower_right(L, n))[0]
        np.testing.assert_allclose(out[t0:t1], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_row_i_equals_decode_over_truncated_sequence():
    rng = np.random.default_rng(3)
    c = _case(rng, [50, 29], [5, 3], Hkv=2, G=4, d=32)
    full = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], 4)
    for b in range(2):
        D = c["q_start"][b + 1] - c["q_start"][b] - 1
        for i in range(D + 1):
            row = c["q_start"][b] + i
            one = verify_attention(c["q"][row:row + 1], c["kc"], c["vc"], c["bt"][b:b + 1],
                                   np.asarray([c["kv_len"][b] - D + i], np.int32),
                                   np.asarray([0, 1], np.int32), 4)
            np.testing.assert_array_equal(one[0], full[row])


def test_page_relabelling_invariance():
    rng = np.random.default_rng(5)
    c = _case(rng, [70, 45], [2, 6], Hkv=2, G=2, d=16)
    out = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], 2)
    pi = rng.permutation(c["kc"].shape[0])
    kc2 = np.empty_like(c["kc"])
    vc2 = np.empty_like(c["vc"])
    kc2[pi] = c["kc"]
    vc2[pi] = c["vc"]
    bt2 = np.where(c["bt"] >= 0, pi[np.maximum(c["bt"], 0)], -1).astype(np.int32)
    out2 = verify_attention(c["q"], kc2, vc2, bt2, c["kv_len"], c["q_start"], 2)
    np.testing.assert_array_equal(out, out2)


def test_constant_values_and_dominant_key():
    rng = np.random.default_rng(9)
    c = _case(rng, [40], [3], Hkv=1, G=2, d=16)
    vconst = _rand_bits(rng, (16,))
    vc = c["vc"].copy()
    vc[:, 0, :, :] = vconst[:, None]     # every key's value row is vconst (pages are d-major)
    out = verify_attention(c["q"], c["kc"], vc, c["bt"], c["kv_len"], c["q_start"], 2)
    np.testing.assert_allclose(out[0], np.broadcast_to(bf16_bits_to_f64(vconst), out[0].shape),
                               rtol=0, atol=1e-14)
    # make key 5 dominate: K_5 = 64 * q (bf16-exact scaling by a power of two)
    kc = c["kc"].copy()
    qrow = bf16_bits_to_f64(c["q"][0, 0])
    k5 = torch.from_numpy((64.0 * qrow).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    page, slot = c["bt"][0, 5 // 16], 5 % 16
    kc[page, 0, slot, :] = k5.view(np.uint16)
    out = verify_attention(c["q"], kc, c["vc"], c["bt"], c["kv_len"], c["q_start"], 2)
    v5 = bf16_bits_to_f64(c["vc"][page, 0, :, slot])
    np.testing.assert_allclose(out[0, 0], v5, rtol=0, atol=1e-9)


def test_vanishing_scale_gives_mean_of_visible_values():
    rng = np.random.default_rng(21)
    c = _case(rng, [37], [4], Hkv=1, G=1, d=8)
    out = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], 1, scale=1e-300)
    V = bf16_bits_to_f64(c["dense_v"][0][0])
    for i in range(5):
        P = 37 - 5 + i
        np.testing.assert_allclose(out[i, 0], V[: P + 1].mean(0), rtol=0, atol=1e-14)


def test_sequence_shorter_than_its_block_gives_zero_rows():
    rng = np.random.default_rng(2)
    c = _case(rng, [3], [5], Hkv=1, G=2, d=8)     # rows 0..2 see nothing (P < 0)
    out = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], 2)
    assert np.all(out[:3] == 0.0)
    # row 3 sees key 0 only -> its value; row 5 sees keys 0..2
    v0 = bf16_bits_to_f64(c["dense_v"][0][0, 0])
    np.testing.assert_allclose(out[3, 0], v0, atol=1e-15, rtol=0)
    assert np.all(np.isfinite(out))


def test_units_subset_matches_full():
    rng = np.random.default_rng(4)
    c = _case(rng, [30, 31, 32], [1, 2, 3], Hkv=2, G=2, d=16)
    full = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], 2, workers=3)
    part = verify_attention(c["q"], c["kc"], c["vc"], c["bt"], c["kv_len"], c["q_start"], 2, units=[(1, 1)])
    t0, t1 = c["q_start"][1], c["q_start"][2]
    np.testing.assert_array_equal(part[t0:t1, 2:4], full[t0:t1, 2:4])
    assert np.isnan(part[0]).all()


def test_rejects_bad_page_ids():
    rng = np.random.default_rng(1)
    c = _case(rng, [20], [1], Hkv=1, G=1, d=8)
    bt = c["bt"].copy()
    bt[0, 1] = c["kc"].shape[0]
    with pytest.raises(ValueError):
        verify_attention(c["q"], c["kc"], c["vc"], bt, c["kv_len"], c["q_start"], 1)


def test_key_major_and_dim_major_v_pages_give_the_same_result():
    """The oracle reads V by (page, head, slot, dimension) from either page
    layout: a cache whose V pages are stored key-major ([P, H, page, d], like K,
    v_layout 'key') gives exactly the output of the same cache stored d-major."""
    rng = np.random.default_rng(11)
    for d, G, kv, drafts in ((64, 2, [40, 17, 300], [3, 0, 7]), (128, 4, [1000, 33], [15, 2])):
        B = len(kv)
        q_start = np.concatenate([[0], np.cumsum(np.asarray(drafts) + 1)]).astype(np.int32)
        T = int(q_start[-1])
        npg = [-(-n // 16) for n in kv]
        P = sum(npg) + 3
        perm = rng.permutation(P).astype(np.int32)
        bt = np.zeros((B, max(npg)), np.int32)
        o = 0
        for b in range(B):
            bt[b, :npg[b]] = perm[o:o + npg[b]]
            o += npg[b]
        k = rng.integers(0, 1 << 16, size=(P, 2, 16, d), dtype=np.uint32).astype(np.uint16) & 0xBFFF
        v_dm = rng.integers(0, 1 << 16, size=(P, 2, d, 16), dtype=np.uint32).astype(np.uint16) & 0xBFFF
        q = rng.integers(0, 1 << 16, size=(T, 2 * G, d), dtype=np.uint32).astype(np.uint16) & 0xBFFF
        args = dict(q_bits=q, k_bits=k, block_table=bt, kv_len=np.asarray(kv, np.int32), q_start=q_start, group=G)
        a = verify_attention(v_bits=v_dm, **args)
        b_ = verify_attention(v_bits=np.ascontiguousarray(v_dm.transpose(0, 1, 3, 2)), v_layout="key", **args)
        np.testing.assert_array_equal(a, b_)
