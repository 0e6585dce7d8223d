"""Pins for the attention oracle: dense equivalence, closed forms, literal masks.

The attention consumer is not printed on any page; its definition is the plain
reading stated in the oracle's docstring. These tests pin that definition to a
library routine (torch's scaled_dot_product_attention in fp64 when every tile is
kept, the case the selection page's ``force`` switch exists for), to closed
forms, and to a literal token-level mask.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _qkv(B, Hq, Hkv, S, D, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, S, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, S, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, S, D, generator=g).to(dtype)
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (6, 1)])
def test_force_budget_one_equals_dense_sdpa(causal, Hq, Hkv):
    """budget 1.0 with force keeps every tile, so attention equals plain SDPA (fp64)."""
    B, S, D, bq, bkv = 2, 200, 32, 64, 32
    q, k, v = _qkv(B, Hq, Hkv, S, D, seed=Hq * 10 + Hkv + causal)
    sel = oracle.select_blocks(q, k, 1.0, bq, bkv, False, True)
    assert np.all(sel["keep"] == 1)
    out, lse = oracle.attention(q, k, v, sel["keep"], bq, bkv, causal)
    g = Hq // Hkv
    kr = k.double().repeat_interleave(g, dim=1)
    vr = v.double().repeat_interleave(g, dim=1)
    ref = F.scaled_dot_product_attention(q.double(), kr, vr, is_causal=causal)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12
    logits = (q.double() @ kr.transpose(-1, -2)) / math.sqrt(D)
    if causal:
        logits = logits.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    ref_lse = torch.logsumexp(logits, dim=-1)
    assert np.max(np.abs(lse - ref_lse.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_form(causal):
    """q = 0: every visible key has logit 0, so LSE = ln(#visible) and O = mean of visible v."""
    B, H, S, D, bq, bkv = 1, 2, 192, 16, 64, 32
    _, k, v = _qkv(B, H, H, S, D, seed=3)
    q = torch.zeros(B, H, S, D)
    rng = np.random.default_rng(0)
    keep = (rng.random((B, H, 3, 6)) < 0.5).astype(np.int8)
    keep |= oracle.diagonal_blocks(3, 6, bq, bkv)[None, None].astype(np.int8)
    out, lse = oracle.attention(q, k, v, keep, bq, bkv, causal)
    cnt = oracle.visible_key_counts(keep, bq, bkv, S, S, causal)
    assert np.allclose(lse, np.log(cnt), atol=1e-12, rtol=0)
    for h in range(H):
        for t in range(0, S, 7):
            tiles = np.nonzero(keep[0, h, t // bq])[0]
            idx = [u for j in tiles for u in range(j * bkv, min((j + 1) * bkv, S))
                   if (not causal or u <= t)]
            want = v[0, h, idx].double().mean(0).numpy()
            assert np.allclose(out[0, h, t], want, atol=1e-12, rtol=0)


def test_causal_first_token_sees_only_itself():
    B, H, S, D, bq, bkv = 1, 1, 128, 32, 64, 32
    q, k, v = _qkv(B, H, H, S, D, seed=5)
    keep = np.ones((1, 1, 2, 4), np.int8)
    out, lse = oracle.attention(q, k, v, keep, bq, bkv, True)
    assert np.allclose(out[0, 0, 0], v[0, 0, 0].double().numpy(), atol=1e-14, rtol=0)
    want = float((q[0, 0, 0].double() @ k[0, 0, 0].double()) / math.sqrt(D))
    assert abs(lse[0, 0, 0] - want) < 1e-12


def test_identical_keys_give_uniform_weights():
    B, H, S, D, bq, bkv = 1, 1, 128, 16, 64, 32
    q, _, v = _qkv(B, H, H, S, D, seed=8)
    k = torch.randn(1, 1, 1, D).repeat(1, 1, S, 1)
    keep = np.zeros((1, 1, 2, 4), np.int8)
    keep[0, 0, 0, [0, 2]] = 1
    keep[0, 0, 1, [1, 3]] = 1
    out, lse = oracle.attention(q, k, v, keep, bq, bkv, False)
    for t in (0, 17, 63):
        idx = list(range(0, 32)) + list(range(64, 96))
        assert np.allclose(out[0, 0, t], v[0, 0, idx].double().mean(0).numpy(), atol=1e-12)
        logit = float(q[0, 0, t].double() @ k[0, 0, 0].double()) / math.sqrt(D)
        assert abs(lse[0, 0, t] - (logit + math.log(64))) < 1e-12


def test_empty_row_gives_zero_and_minus_inf():
    """Dropping a row's diagonal under causal leaves early queries with nothing: O = 0, LSE = -inf."""
    B, H, S, D, bq, bkv = 1, 1, 128, 16, 64, 32
    q, k, v = _qkv(B, H, H, S, D, seed=9)
    keep = np.zeros((1, 1, 2, 4), np.int8)
    keep[0, 0, 0, 1] = 1  # tokens 32..63 only: queries 0..31 see nothing under causal
    keep[0, 0, 1, 2] = 1
    out, lse = oracle.attention(q, k, v, keep, bq, bkv, True)
    assert np.all(out[0, 0, :32] == 0) and np.all(np.isneginf(lse[0, 0, :32]))
    assert np.all(np.isfinite(lse[0, 0, 32:]))


@pytest.mark.parametrize("causal", [False, True])
def test_gathered_equals_literal_mask_on_tiny_workload(causal):
    """The per-row gathered oracle equals the literal S x S mask (tiny fp32 workload shape)."""
    w = synth.workload("tiny_causal_f32")
    inp = synth.make_inputs(w)
    sel = oracle.select_blocks(inp.q, inp.k, w.budget, w.block_q, w.block_kv, w.head_shared)
    a_o, a_l = oracle.attention(inp.q, inp.k, inp.v, sel["keep"], w.block_q, w.block_kv, causal)
    b_o, b_l = oracle.attention_dense_literal(inp.q, inp.k, inp.v, sel["keep"], w.block_q,
                                              w.block_kv, causal)
    assert np.max(np.abs(a_o - b_o)) < 1e-12
    assert np.max(np.abs(a_l - b_l)) < 1e-12


def test_gathered_equals_literal_mask_gqa_headshared_tails():
    """Same check with GQA, head-shared keep, pins, drops and ragged tails."""
    B, Hq, Hkv, S, D, bq, bkv = 2, 4, 2, 300, 16, 64, 32
    q, k, v = _qkv(B, Hq, Hkv, S, D, seed=21, dtype=torch.bfloat16)
    nq, nk = 5, 10
    pins = np.zeros((1, 1, nq, nk), np.int8)
    pins[..., 0] = 1
    drops = np.zeros((2, 1, nq, nk), np.int8)
    drops[1, 0, 4, 2] = 1
    sel = oracle.select_blocks(q, k, 0.3, bq, bkv, True, False, pins, drops)
    assert sel["keep"].shape == (2, 1, nq, nk)
    for causal in (False, True):
        a_o, a_l = oracle.attention(q, k, v, sel["keep"], bq, bkv, causal)
        b_o, b_l = oracle.attention_dense_literal(q, k, v, sel["keep"], bq, bkv, causal)
        assert np.max(np.abs(a_o - b_o)) < 1e-12
        assert np.max(np.abs(a_l - b_l)) < 1e-12


def test_gathered_equals_literal_mask_scaled_mha_workload():
    """The MHA 8k workload recipe at a reduced length (2 heads, S 1024) against the literal mask."""
    w = synth.workload("mha_bf16_s8k").scaled(Hq=2, Hkv=2, S=1024)
    inp = synth.make_inputs(w)
    sel = oracle.select_blocks(inp.q, inp.k, w.budget, w.block_q, w.block_kv, w.head_shared)
    a_o, a_l = oracle.attention(inp.q, inp.k, inp.v, sel["keep"], w.block_q, w.block_kv, False)
    b_o, b_l = oracle.attention_dense_literal(inp.q, inp.k, inp.v, sel["keep"], w.block_q,
                                              w.block_kv, False)
    assert np.max(np.abs(a_o - b_o)) < 1e-12
    assert np.max(np.abs(a_l - b_l)) < 1e-12


def test_row_subset_matches_full():
    B, H, S, D, bq, bkv = 1, 2, 256, 16, 64, 32
    q, k, v = _qkv(B, H, H, S, D, seed=4)
    sel = oracle.select_blocks(q, k, 0.3, bq, bkv, False, True)
    full_o, full_l = oracle.attention(q, k, v, sel["keep"], bq, bkv, True)
    rows = [(0, 1, 2), (0, 0, 3)]
    o, l = oracle.attention(q, k, v, sel["keep"], bq, bkv, True, rows=rows)
    for b, h, i in rows:
        sl = slice(i * bq, (i + 1) * bq)
        assert np.array_equal(o[b, h, sl], full_o[b, h, sl])
        assert np.array_equal(l[b, h, sl], full_l[b, h, sl])
