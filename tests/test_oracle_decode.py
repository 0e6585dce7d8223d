"""Pins for the decode oracle.

* Reduction to the page's function on the full sequence: the last query tiles
  of a full select_blocks (tiles aligned at 0) are exactly the decode
  selection of those tokens at their absolute position, since the pooled
  queries, pooled keys, diagonal and candidates coincide.
* With every tile kept, decode attention equals the last rows of full causal
  SDPA over the cache (the KV-cache identity), checked against torch in fp64.
* One query token at the end of the cache: its diagonal is exactly the kv tile
  holding its position.
* A cache longer than the valid length: tokens past the length never matter.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _seq(B, Hq, Hkv, S, D, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, Hq, S, D, generator=g).to(dtype), torch.randn(B, Hkv, S, D, generator=g).to(dtype),
            torch.randn(B, Hkv, S, D, generator=g).to(dtype))


@pytest.mark.parametrize("shared", [False, True])
def test_decode_select_equals_last_tiles_of_full_select(shared):
    B, Hq, Hkv, S, D, bq, bkv = 1, 4, 2, 1024, 32, 128, 64
    q, k, _ = _seq(B, Hq, Hkv, S, D, seed=3)
    full = oracle.select_blocks(q, k, 0.3, bq, bkv, shared, True)
    for first_tile in (7, 5, 0):
        pos0 = first_tile * bq
        dec = oracle.decode_select(q[:, :, pos0:], k, S, pos0, 0.3, bq, bkv, shared, True)
        assert np.array_equal(dec["keep"], full["keep"][:, :, first_tile:])


@pytest.mark.parametrize("n,bq", [(1, 128), (3, 128), (64, 32), (130, 64)])
def test_decode_attention_all_kept_equals_causal_sdpa_tail(n, bq):
    B, Hq, Hkv, S, D, bkv = 1, 4, 2, 700, 32, 64
    q, k, v = _seq(B, Hq, Hkv, S, D, seed=n + bq)
    pos0 = S - n
    nq, nk = -(-n // bq), -(-S // bkv)
    keep = np.ones((1, 1, nq, nk), np.int8)
    out, lse = oracle.decode_attention(q[:, :, pos0:], k, v, S, pos0, keep, bq, bkv)
    g = Hq // Hkv
    kr, vr = k.double().repeat_interleave(g, 1), v.double().repeat_interleave(g, 1)
    ref = F.scaled_dot_product_attention(q.double(), kr, vr, is_causal=True)[:, :, pos0:]
    assert np.max(np.abs(out - ref.numpy())) < 1e-12
    logits = (q.double() @ kr.transpose(-1, -2)) / np.sqrt(D)
    logits = logits.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(logits, -1)[:, :, pos0:].numpy())) < 1e-12


@pytest.mark.parametrize("L,bkv", [(700, 64), (640, 64), (641, 64), (1, 64), (1000, 32)])
def test_single_token_diagonal_is_its_own_tile(L, bkv):
    nk = -(-L // bkv)
    d = oracle.diagonal_blocks(1, nk, 128, bkv, q_offset=L - 1)
    want = np.zeros((1, nk), bool)
    want[0, (L - 1) // bkv:] = True   # tiles from its own up to the end of its (unclipped) query tile
    want[0, :] &= np.arange(nk) * bkv < L - 1 + 128
    assert np.array_equal(d, want)
    assert d[0, (L - 1) // bkv] and not d[0, :(L - 1) // bkv].any()


def test_cache_tail_beyond_length_is_ignored():
    B, Hq, Hkv, S, D, bq, bkv = 1, 2, 1, 512, 32, 128, 64
    q, k, v = _seq(B, Hq, Hkv, S, D, seed=9)
    L = 450
    k2, v2 = k.clone(), v.clone()
    k2[:, :, L:] = 1e6
    v2[:, :, L:] = float("nan")
    qn = q[:, :, L - 2:L]
    a = oracle.decode_select(qn, k, L, L - 2, 0.5, bq, bkv, False, True)
    b = oracle.decode_select(qn, k2, L, L - 2, 0.5, bq, bkv, False, True)
    assert np.array_equal(a["keep"], b["keep"])
    oa, la = oracle.decode_attention(qn, k, v, L, L - 2, a["keep"], bq, bkv)
    ob, lb = oracle.decode_attention(qn, k2, v2, L, L - 2, a["keep"], bq, bkv)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    assert torch.equal(oracle.decode_pool(k, L, bkv), oracle.pool_blocks(k[:, :, :L], bkv))
