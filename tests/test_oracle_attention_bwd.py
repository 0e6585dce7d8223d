"""Pins for the attention-gradient oracle.

The gradient oracle is written out by hand (dP, Delta, dS). It is pinned to
routes that share none of that code:
* torch autograd of scaled_dot_product_attention in fp64 when every tile is
  kept (force with budget 1, the selection page's dense switch);
* torch autograd through a literal token-level masked softmax, for random
  keep patterns with empty query rows;
* central finite differences of the forward oracle on a tiny case;
* closed forms: a constant V gives zero dQ and dK, and each kv head's dV sums
  to the sum of dO over its queries that see any key.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention_bwd import attention_backward


def _qkvd(B, Hq, Hkv, S, D, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, S, D, generator=g, dtype=torch.float64).to(dtype)
    k = torch.randn(B, Hkv, S, D, generator=g, dtype=torch.float64).to(dtype)
    v = torch.randn(B, Hkv, S, D, generator=g, dtype=torch.float64).to(dtype)
    do = torch.randn(B, Hq, S, D, generator=g, dtype=torch.float64).to(dtype)
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (6, 1)])
def test_dense_equals_autograd_sdpa(causal, Hq, Hkv):
    B, S, D, bq, bkv = 2, 150, 16, 64, 32
    q, k, v, do = _qkvd(B, Hq, Hkv, S, D, seed=Hq * 3 + Hkv + 7 * causal)
    sel = oracle.select_blocks(q.float(), k.float(), 1.0, bq, bkv, False, True)
    assert np.all(sel["keep"] == 1)
    dq, dk, dv = attention_backward(q, k, v, do, sel["keep"], bq, bkv, causal)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    g = Hq // Hkv
    out = F.scaled_dot_product_attention(qa, ka.repeat_interleave(g, 1), va.repeat_interleave(g, 1),
                                         is_causal=causal)
    out.backward(do)
    for got, ref in ((dq, qa.grad), (dk, ka.grad), (dv, va.grad)):
        assert np.max(np.abs(got - ref.numpy())) < 1e-11


def _literal_masked_attention(q, k, v, keep, bq, bkv, causal):
    """Token-level masked attention written with torch ops so autograd can differentiate it."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    keep = torch.as_tensor(np.asarray(keep) != 0)
    tq = torch.arange(S) // bq
    tk = torch.arange(S) // bkv
    outs = []
    for b in range(B):
        per_head = []
        for h in range(Hq):
            km = keep[b if keep.shape[0] == B else 0, h if keep.shape[1] == Hq else 0]
            vis = km[tq[:, None], tk[None, :]]
            if causal:
                vis = vis & (torch.arange(S)[None, :] <= torch.arange(S)[:, None])
            logits = (q[b, h] @ k[b, h // g].T) / math.sqrt(D)
            shift = torch.where(vis, logits, torch.full_like(logits, -torch.inf)).max(dim=1).values
            shift = torch.where(torch.isfinite(shift), shift, torch.zeros_like(shift)).detach()
            w = torch.exp(logits - shift[:, None]) * vis
            tot = w.sum(dim=1, keepdim=True)
            per_head.append((w @ v[b, h // g]) / torch.where(tot > 0, tot, torch.ones_like(tot)))
        outs.append(torch.stack(per_head))
    return torch.stack(outs)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shared", [False, True])
def test_random_keep_equals_autograd_of_literal_mask(causal, shared):
    B, Hq, Hkv, S, D, bq, bkv = 2, 4, 2, 200, 16, 64, 32
    nq, nk = -(-S // bq), -(-S // bkv)
    q, k, v, do = _qkvd(B, Hq, Hkv, S, D, seed=11 + causal + 2 * shared)
    rng = np.random.default_rng(3 + causal)
    keep = (rng.random((B, 1 if shared else Hq, nq, nk)) < 0.4).astype(np.int8)
    keep[0, 0, 1, :] = 0                      # an empty query tile
    dq, dk, dv = attention_backward(q, k, v, do, keep, bq, bkv, causal)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = _literal_masked_attention(qa, ka, va, keep, bq, bkv, causal)
    ref_out, _ = oracle.attention(q, k, v, keep, bq, bkv, causal)
    assert np.max(np.abs(out.detach().numpy() - ref_out)) < 1e-12
    out.backward(do)
    for got, ref in ((dq, qa.grad), (dk, ka.grad), (dv, va.grad)):
        assert np.max(np.abs(got - ref.numpy())) < 1e-11
    assert np.all(dq[0, 0, bq:2 * bq] == 0)  # the empty tile's queries get no gradient


def test_central_finite_differences():
    B, Hq, Hkv, S, D, bq, bkv = 1, 2, 1, 40, 8, 16, 8
    nq, nk = -(-S // bq), -(-S // bkv)
    q, k, v, do = _qkvd(B, Hq, Hkv, S, D, seed=5)
    keep = (np.random.default_rng(9).random((B, Hq, nq, nk)) < 0.6).astype(np.int8)
    keep |= oracle.diagonal_blocks(nq, nk, bq, bkv)[None, None].astype(np.int8)
    dq, dk, dv = attention_backward(q, k, v, do, keep, bq, bkv, True)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, keep, bq, bkv, True)
        return float((o * do.numpy()).sum())

    h = 1e-6
    rng = np.random.default_rng(1)
    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in t.shape)
            tp, tm = t.clone(), t.clone()
            tp[idx] += h
            tm[idx] -= h
            plus = {"q": q, "k": k, "v": v}
            minus = dict(plus)
            plus[name], minus[name] = tp, tm
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_closed_forms(causal):
    """v_u = c for all u: O_t = c whatever the weights, so dQ = dK = 0, and
    sum_u dV[u] = sum over queries that see a key of dO_t (rows of P sum to 1)."""
    B, Hq, Hkv, S, D, bq, bkv = 1, 4, 2, 160, 8, 32, 32
    nq, nk = -(-S // bq), -(-S // bkv)
    q, k, _, do = _qkvd(B, Hq, Hkv, S, D, seed=21)
    c = torch.randn(D, dtype=torch.float64)
    v = c.expand(B, Hkv, S, D).clone()
    rng = np.random.default_rng(4)
    keep = (rng.random((B, Hq, nq, nk)) < 0.5).astype(np.int8)
    keep[0, 1, 2] = 0
    dq, dk, dv = attention_backward(q, k, v, do, keep, bq, bkv, causal)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    cnt = oracle.visible_key_counts(keep, bq, bkv, S, S, causal)        # (1, Hq, S)
    seen = cnt[0] > 0
    for g in range(Hkv):
        want = sum((do[0, h].numpy() * seen[h][:, None]).sum(0) for h in range(2 * g, 2 * g + 2))
        assert np.allclose(dv[0, g].sum(0), want, atol=1e-10, rtol=0)


def test_sampled_outputs_equal_full():
    B, Hq, Hkv, S, D, bq, bkv = 1, 4, 2, 256, 16, 64, 32
    nq, nk = -(-S // bq), -(-S // bkv)
    q, k, v, do = _qkvd(B, Hq, Hkv, S, D, seed=2)
    keep = (np.random.default_rng(2).random((B, Hq, nq, nk)) < 0.5).astype(np.int8)
    dq, dk, dv = attention_backward(q, k, v, do, keep, bq, bkv, True)
    rows = [(0, 1, 2), (0, 3, 0)]
    tiles = [(0, 0, 3), (0, 1, 7)]
    sq, sk, sv = attention_backward(q, k, v, do, keep, bq, bkv, True, rows=rows, kv_tiles=tiles)
    for b, h, i in rows:
        assert np.array_equal(sq[b, h, i * bq:(i + 1) * bq], dq[b, h, i * bq:(i + 1) * bq])
    for b, g, j in tiles:
        sl = slice(j * bkv, (j + 1) * bkv)
        assert np.allclose(sk[b, g, sl], dk[b, g, sl], atol=1e-13, rtol=0)
        assert np.allclose(sv[b, g, sl], dv[b, g, sl], atol=1e-13, rtol=0)
    assert np.isnan(sq[0, 0, 0, 0]) and np.isnan(sk[0, 0, 0, 0])
