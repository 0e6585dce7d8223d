"""Checks of the seeded workload generators (structure only, no method arithmetic)."""
import numpy as np
import torch

import synth


def test_deterministic_and_shapes():
    w = synth.workload("tiny_causal_f32")
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    assert a.q.shape == (1, 2, 512, 64) and a.q.dtype == torch.float32
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    c = synth.make_inputs(w, seed=5)
    assert not torch.equal(a.q, c.q)


def test_bf16_cast():
    w = synth.workload("mha_bf16_s8k").scaled(Hq=2, Hkv=2, S=256)
    inp = synth.make_inputs(w)
    assert inp.q.dtype == torch.bfloat16 and inp.k.is_contiguous()


def test_morton_tiles_are_square_patches():
    y, x = synth.morton_grid_coords(128, 256)
    assert sorted(zip(y.tolist(), x.tolist())) == [(a, c) for a in range(128) for c in range(256)]
    for t in (0, 1, 77, 511):  # a kv tile of 64 tokens is an 8 x 8 patch
        ys, xs = y[t * 64:(t + 1) * 64], x[t * 64:(t + 1) * 64]
        assert ys.max() - ys.min() == 7 and xs.max() - xs.min() == 7
    for t in (0, 5, 255):  # a query tile of 128 tokens is 8 rows x 16 columns
        ys, xs = y[t * 128:(t + 1) * 128], x[t * 128:(t + 1) * 128]
        assert ys.max() - ys.min() == 7 and xs.max() - xs.min() == 15
    # the Z-order index of (y, x) interleaves x in the even bits and y in the odd bits
    assert (y[2], x[2]) == (1, 0) and (y[1], x[1]) == (0, 1) and (y[1 << 14], x[1 << 14]) == (0, 128)


def test_drops_avoid_intersecting_and_pinned_tiles():
    w = synth.workload("long_causal_gqa_bf16_s128k").scaled(Hq=2, Hkv=1, S=8192)
    inp = synth.make_inputs(w)
    nq, nk = w.nq, w.nk
    inter = synth.tile_ranges_intersect(nq, nk, w.block_q, w.block_kv)
    assert inp.pins.shape == (1, 1, nq, nk) and np.all(inp.pins[..., 0] == 1)
    assert inp.pins.sum() == nq
    d = inp.drops[0, 0] != 0
    assert not np.any(d & inter) and not np.any(d[:, 0])
    eligible = (~inter).sum() - (inp.pins[0, 0, :, 0] != 0).sum() + inter[:, 0].sum()
    assert d.sum() == int(round(0.01 * eligible))


def test_long_context_drop_count_matches_recipe():
    """At NQ 1024 x NK 2048, 1% of the 2,094,081 eligible tiles is 20,941."""
    nq, nk = 1024, 2048
    inter = synth.tile_ranges_intersect(nq, nk, 128, 64)
    eligible = ~inter
    eligible[:, 0] = False
    assert eligible.sum() == 2094081
    assert int(round(0.01 * eligible.sum())) == 20941


def test_cluster_keys_share_tile_centres():
    w = synth.workload("long_causal_gqa_bf16_s128k").scaled(Hq=1, Hkv=1, S=2048, clusters=4)
    inp = synth.make_inputs(w)
    k = inp.k[0, 0].float()
    means = k.reshape(-1, 64, 128).mean(1)
    # pooled tiles land near one of 4 centres: pairwise distances are bimodal,
    # about 2 (same centre, noise of a 64-token mean) or about 16 (two centres)
    dist = torch.cdist(means, means)
    assert (dist < 5).float().mean() > 0.2
    assert ((dist > 5) & (dist < 8)).float().sum() == 0
