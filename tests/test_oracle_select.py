"""Pins for the selection oracle: closed forms, invariants, brute force.

Each test checks the oracle against something other than itself: a closed form
the page fixes, an invariant the page states, a brute-force enumeration, or an
independent re-derivation of IEEE fp32 arithmetic. Pages cited by title; the
selection page is "automatic/modules/attention/sparse/selector.py".
"""
import itertools
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import select as osel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fl32(x: float) -> float:
    """Round a double to the nearest fp32 (IEEE, ties to even) via struct."""
    return struct.unpack("f", struct.pack("f", x))[0]


# ---------------------------------------------------------------- geometry

def test_block_count_closed_form():
    assert oracle.block_count(512, 64) == 8
    assert oracle.block_count(100, 64) == 2
    assert oracle.block_count(1, 64) == 1
    assert oracle.block_count(64, 64) == 1
    assert oracle.block_count(65, 64) == 2
    assert oracle.block_count(0, 64) == 0


@pytest.mark.parametrize("bq,bkv,nq,nk", [(128, 64, 9, 18), (64, 32, 8, 16), (64, 64, 5, 5),
                                          (32, 64, 8, 4), (96, 64, 5, 8), (128, 48, 4, 11)])
def test_diagonal_closed_form(bq, bkv, nq, nk):
    """Row i keeps kv tiles floor(i*bq/bkv) .. ceil((i+1)*bq/bkv)-1, clipped to NK."""
    d = oracle.diagonal_blocks(nq, nk, bq, bkv)
    for i in range(nq):
        lo = (i * bq) // bkv
        hi = -(-((i + 1) * bq) // bkv) - 1
        want = np.zeros(nk, bool)
        want[lo:min(hi, nk - 1) + 1] = True
        assert np.array_equal(d[i], want), (i, d[i], want)
    if bq == 2 * bkv and nk >= 2 * nq:
        assert np.all(d.sum(1) == 2)


# ---------------------------------------------------------------- pooling

def test_pool_constant_exact():
    x = torch.full((1, 2, 100, 8), 0.375)
    p = oracle.pool_blocks(x, 64)
    assert p.shape == (1, 2, 2, 8)
    assert torch.all(p == 0.375)


def test_pool_ramp_midpoint_and_tail():
    """x[t] = t gives the midpoint (start + end - 1) / 2 of each tile, tail included."""
    S, blk = 300, 64
    x = torch.arange(S, dtype=torch.float32)[None, None, :, None].repeat(1, 1, 1, 4)
    p = oracle.pool_blocks(x, blk)
    for i in range(p.shape[-2]):
        lo, hi = i * blk, min((i + 1) * blk, S)
        assert torch.all(p[0, 0, i] == (lo + hi - 1) / 2), (i, p[0, 0, i])
    # the tail tile (tokens 256..299, 44 of them) is averaged over its 44 tokens
    assert p[0, 0, -1, 0].item() == (256 + 299) / 2


def test_pool_short_sequence_single_tile():
    x = torch.randn(1, 1, 10, 16, dtype=torch.float64).to(torch.float32)
    p = oracle.pool_blocks(x, 64)
    assert p.shape == (1, 1, 1, 16)
    ref = x.to(torch.float64).mean(dim=-2)
    assert torch.allclose(p[0, 0, 0].double(), ref[0, 0], rtol=0, atol=1e-6)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pool_matches_fp64_mean_within_fp32_bound(dtype):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(2, 3, 333, 32, generator=g).to(dtype)
    p = oracle.pool_blocks(x, 64).double()
    for i in range(p.shape[-2]):
        seg = x[..., i * 64:min((i + 1) * 64, 333), :].double()
        ref = seg.mean(dim=-2)
        bound = seg.shape[-2] * 2 ** -24 * seg.abs().mean(dim=-2) * 2 + 1e-30
        assert torch.all((p[..., i, :] - ref).abs() <= bound)


# ---------------------------------------------------------------- scores

def _tile_constant(vectors, block, seq):
    """A (H, seq, D) tensor whose tile t holds vectors[:, t] on every token."""
    h, n, d = vectors.shape
    out = torch.empty(h, seq, d)
    for t in range(n):
        out[:, t * block:min((t + 1) * block, seq)] = vectors[:, t:t + 1]
    return out[None]


def test_scores_one_hot():
    """Pooled q = e_a(i), pooled k = e_b(j) gives s[i, j] = [a(i) == b(j)]."""
    D, bq, bkv, S = 8, 32, 16, 128
    a = [3, 0, 5, 3]
    b = [0, 3, 1, 5, 5, 2, 3, 7]
    eq = torch.zeros(1, 4, D)
    ek = torch.zeros(1, 8, D)
    for i, ai in enumerate(a):
        eq[0, i, ai] = 1
    for j, bj in enumerate(b):
        ek[0, j, bj] = 1
    q = _tile_constant(eq, bq, S)
    k = _tile_constant(ek, bkv, S)
    s = oracle.score_blocks(q, k, bq, bkv, head_shared=False)
    want = np.array([[1.0 if ai == bj else 0.0 for bj in b] for ai in a], np.float32)
    assert np.array_equal(s[0, 0], want)


def test_scores_gqa_kv_head_mapping():
    """Query head h scores against kv head h // (Hq/Hkv), not h % Hkv."""
    D, bq, bkv, S, Hq, Hkv = 4, 16, 16, 32, 6, 2
    q = torch.zeros(1, Hq, S, D)
    q[..., 0] = 1.0
    k = torch.zeros(1, Hkv, S, D)
    k[0, 0, :, 0] = 2.0
    k[0, 1, :, 0] = 5.0
    s = oracle.score_blocks(q, k, bq, bkv, head_shared=False)
    assert s.shape == (1, Hq, 2, 2)
    for h in range(Hq):
        assert np.all(s[0, h] == (2.0 if h < 3 else 5.0)), h


def test_scores_head_shared_is_product_of_means():
    """head_shared scores mean_h(q) . mean_g(k), which differs from mean_h(q_h . k_h)."""
    D, S, blk = 2, 16, 16
    q = torch.zeros(1, 2, S, D)
    k = torch.zeros(1, 2, S, D)
    q[0, 0, :, 0] = 1.0
    q[0, 1, :, 1] = 3.0
    k[0, 0, :, 0] = 2.0
    k[0, 1, :, 1] = 4.0
    s = oracle.score_blocks(q, k, blk, blk, head_shared=True)
    # mean q = (0.5, 1.5), mean k = (1, 2): 0.5 + 3 = 3.5 (mean of per-head scores would be 7)
    assert s.shape == (1, 1, 1, 1)
    assert s[0, 0, 0, 0] == 3.5


def test_scores_within_fp32_error_bound():
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 2, 256, 64, generator=g)
    k = torch.randn(1, 2, 256, 64, generator=g)
    s = oracle.score_blocks(q, k, 64, 32, head_shared=False).astype(np.float64)
    pq = oracle.pool_blocks(q, 64).double().numpy()
    pk = oracle.pool_blocks(k, 32).double().numpy()
    exact = pq @ np.swapaxes(pk, -1, -2)
    mag = np.abs(pq) @ np.swapaxes(np.abs(pk), -1, -2)
    assert np.all(np.abs(s - exact) <= 64 * 2 ** -24 * mag * 1.01 + 1e-30)


# ---------------------------------------------------------------- plan

def test_keep_per_row_fl32_golden():
    rows = []
    with open(os.path.join(GOLDEN, "keep_per_row_fl32.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                b, c, kk = line.split()
                rows.append((float(b), int(c), int(kk)))
    assert len(rows) >= 8
    for b, c, kk in rows:
        assert int(oracle.keep_per_row(np.array([c]), b)[0]) == kk, (b, c)
        # independent re-derivation of the IEEE fp32 product
        assert math.ceil(fl32(fl32(float(c)) * fl32(b))) == kk


def test_keep_per_row_fl32_exhaustive_against_struct():
    for b in (0.30, 0.25, 0.15, 0.10, 0.05, 0.7):
        c = np.arange(0, 4097)
        got = oracle.keep_per_row(c, b)
        want = np.array([math.ceil(fl32(fl32(float(x)) * fl32(b))) for x in c])
        assert np.array_equal(got, want), b


def _random_masks(rng, shape4, p_pin=0.1, p_drop=0.1):
    pins = (rng.random(shape4) < p_pin).astype(np.int8)
    drops = (rng.random(shape4) < p_drop).astype(np.int8)
    return pins, drops


@pytest.mark.parametrize("pin_shape,drop_shape", [((1, 1), (1, 1)), ((2, 1), (1, 3)), ((2, 3), (2, 3))])
def test_plan_and_select_invariants(pin_shape, drop_shape):
    """|keep_r| = |must_r minus forb_r| + min(k_r, c_r); must minus forb kept; forb never kept."""
    rng = np.random.default_rng(11)
    B, H, S, D, bq, bkv = 2, 3, 250, 16, 32, 16
    nq, nk = oracle.block_count(S, bq), oracle.block_count(S, bkv)
    pins, _ = _random_masks(rng, pin_shape + (nq, nk))
    _, drops = _random_masks(rng, drop_shape + (nq, nk))
    g = torch.Generator().manual_seed(5)
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    for budget in (0.0, 0.1, 0.3, 0.77):
        sel = oracle.select_blocks(q, k, budget, bq, bkv, False, True, pins, drops)
        keep = sel["keep"] != 0
        must, forb = sel["must"], sel["forbidden"]
        diag = oracle.diagonal_blocks(nq, nk, bq, bkv)
        assert np.all(must >= diag)
        assert np.all(must >= (np.broadcast_to(pins, keep.shape) != 0))
        assert np.array_equal(forb, np.broadcast_to(drops, keep.shape) != 0)
        assert np.all(keep[must & ~forb])
        assert not np.any(keep & forb)
        cand = ~must & ~forb
        assert np.array_equal(sel["c"], cand.sum(-1))
        want = (must & ~forb).sum(-1) + np.minimum(sel["k"], sel["c"])
        assert np.array_equal(keep.sum(-1), want)


def test_drop_wins_over_diagonal_and_pin():
    B, H, S, D, bq, bkv = 1, 1, 128, 8, 32, 32
    nq = nk = 4
    pins = np.zeros((1, 1, nq, nk), np.int8)
    pins[0, 0, 2, 0] = 1
    drops = np.zeros((1, 1, nq, nk), np.int8)
    drops[0, 0, 1, 1] = 1  # a diagonal tile
    drops[0, 0, 2, 0] = 1  # a pinned tile
    g = torch.Generator().manual_seed(1)
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    sel = oracle.select_blocks(q, k, 0.5, bq, bkv, False, True, pins, drops)
    assert sel["keep"][0, 0, 1, 1] == 0
    assert sel["keep"][0, 0, 2, 0] == 0


def test_dense_short_circuit_and_force():
    g = torch.Generator().manual_seed(2)
    q = torch.randn(1, 2, 256, 16, generator=g)
    k = torch.randn(1, 2, 256, 16, generator=g)
    assert oracle.select_blocks(q, k, 1.0, 64, 32, False, False) is None
    sel = oracle.select_blocks(q, k, 1.0, 64, 32, False, True)
    assert np.all(sel["keep"] == 1)
    # a budget below one leaves the sparse path
    assert oracle.select_blocks(q, k, 0.3, 64, 32, False, False) is not None


# ---------------------------------------------------------------- top-k

def test_topk_brute_force_distinct_scores():
    """With distinct scores, the picked set is the unique k-subset of largest total score."""
    g = torch.Generator().manual_seed(9)
    B, H, S, D, bq, bkv = 1, 2, 256, 8, 64, 16  # NQ 4, NK 16
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    for budget in (0.2, 0.36, 0.5):
        sel = oracle.select_blocks(q, k, budget, bq, bkv, False, True)
        s = sel["scores"]
        for h in range(H):
            for i in range(4):
                cand = np.nonzero(~sel["must"][0, h, i])[0]
                vals = s[0, h, i, cand]
                assert len(set(vals.tolist())) == len(vals)
                kk = int(sel["k"][0, h, i])
                best = max(itertools.combinations(range(len(cand)), kk),
                           key=lambda c: float(np.sum(vals[list(c)].astype(np.float64))))
                want = set(cand[list(best)].tolist())
                got = set(np.nonzero(sel["keep"][0, h, i] & ~sel["must"][0, h, i])[0].tolist())
                assert got == want, (budget, h, i)


def test_topk_rank_count_definition_with_ties():
    """j is picked iff #{j' candidate: s_j' > s_j or (s_j' == s_j and j' < j)} < k_r."""
    rng = np.random.default_rng(4)
    for trial in range(200):
        nk = int(rng.integers(1, 20))
        s = rng.integers(-3, 4, size=(1, 1, 1, nk)).astype(np.float32)
        cand = rng.random((1, 1, 1, nk)) < 0.8
        kr = np.array([[[int(rng.integers(0, nk + 2))]]])
        picked, _ = osel.rank_select(s, cand, kr)
        for j in range(nk):
            if not cand[0, 0, 0, j]:
                assert not picked[0, 0, 0, j]
                continue
            ahead = sum(1 for jj in range(nk) if cand[0, 0, 0, jj] and
                        (s[0, 0, 0, jj] > s[0, 0, 0, j] or (s[0, 0, 0, jj] == s[0, 0, 0, j] and jj < j)))
            assert picked[0, 0, 0, j] == (ahead < kr[0, 0, 0]), (trial, j)


def test_topk_all_ties_lowest_index():
    """q = 0 makes every score zero; the picks are the k_r lowest-index candidates."""
    g = torch.Generator().manual_seed(6)
    q = torch.zeros(1, 1, 256, 16)
    k = torch.randn(1, 1, 256, 16, generator=g)
    sel = oracle.select_blocks(q, k, 0.3, 64, 16, False, True)
    s = sel["scores"]
    assert np.all(s == 0)
    for i in range(4):
        cand = np.nonzero(~sel["must"][0, 0, i])[0]
        kk = int(sel["k"][0, 0, i])
        got = np.nonzero(sel["keep"][0, 0, i] & ~sel["must"][0, 0, i])[0]
        assert np.array_equal(got, cand[:kk])


def test_topk_signed_zero_ties_by_index():
    """-0.0 and +0.0 are equal scores: the lower kv index goes first."""
    s = np.array([[[[-0.0, 0.0, -0.0, 1.0, 0.0, -0.0, -1.0]]]], np.float32)
    cand = np.ones_like(s, bool)
    for kk, want in [(1, [3]), (2, [0, 3]), (3, [0, 1, 3]), (4, [0, 1, 2, 3]), (6, [0, 1, 2, 3, 4, 5])]:
        picked, _ = osel.rank_select(s, cand, np.array([[[kk]]]))
        assert np.nonzero(picked[0, 0, 0])[0].tolist() == want


@pytest.mark.parametrize("mq,mk", [(4.0, 1.0), (1.0, 0.25), (2.0 ** 10, 2.0 ** -6)])
def test_topk_invariant_under_power_of_two_scaling(mq, mk):
    g = torch.Generator().manual_seed(8)
    q = torch.randn(1, 3, 512, 32, generator=g)
    k = torch.randn(1, 3, 512, 32, generator=g)
    a = oracle.select_blocks(q, k, 0.3, 64, 32, False, True)
    b = oracle.select_blocks(q * mq, k * mk, 0.3, 64, 32, False, True)
    assert np.array_equal(a["keep"], b["keep"])


def test_topk_invariant_under_row_softmax():
    """Ranking the fp64 softmax of each row picks the same tiles (where no two values collapse)."""
    g = torch.Generator().manual_seed(12)
    q = torch.randn(1, 2, 512, 32, generator=g)
    k = torch.randn(1, 2, 512, 32, generator=g)
    sel = oracle.select_blocks(q, k, 0.3, 64, 32, False, True)
    s = sel["scores"].astype(np.float64) * 20.0
    sm = np.exp(s - s.max(-1, keepdims=True))
    sm /= sm.sum(-1, keepdims=True)
    cand = ~sel["must"]
    p1, _ = osel.rank_select(sel["scores"], cand, sel["k"])
    p2, _ = osel.rank_select(sm, cand, sel["k"])
    for h in range(2):
        for i in range(8):
            if len(set(sm[0, h, i].tolist())) == sm.shape[-1]:
                assert np.array_equal(p1[0, h, i], p2[0, h, i])


def test_near_tie_flag():
    s = np.array([[[[5.0, 3.0, 3.0 * (1 + 5e-6), 1.0, 0.5]]]], np.float64)
    cand = np.ones_like(s, bool)
    _, near = osel.rank_select(s, cand, np.array([[[2]]]))
    assert near[0, 0, 0]
    _, near = osel.rank_select(s, cand, np.array([[[1]]]))
    assert not near[0, 0, 0]
    _, near = osel.rank_select(s, cand, np.array([[[5]]]))  # k = c: nothing left out, no flag
    assert not near[0, 0, 0]


def test_csr_matches_keep():
    rng = np.random.default_rng(3)
    keep = (rng.random((2, 3, 5, 17)) < 0.3).astype(np.int8)
    row_ptr, col_idx = oracle.keep_to_csr(keep)
    flat = keep.reshape(-1, 17)
    assert row_ptr[0] == 0 and row_ptr[-1] == col_idx.size
    for r in range(flat.shape[0]):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(cols) > 0)
        assert np.array_equal(cols, np.nonzero(flat[r])[0])
