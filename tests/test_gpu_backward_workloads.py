"""GPU parity of the attention gradients at full workload sizes, in the launch
configuration the bench times.

The oracle computes sampled outputs one by one: dQ for seeded (batch, head,
query-tile) rows spread over every part of the sequence, and dK / dV for
chosen kv tiles, each the sum over every (query head of the GQA group, query
tile) that keeps the tile. On the 128k workload the kv tiles are the sink
tile 0 (pinned: all 8,192 rows of its kv head read it), the most-read tile of
the middle of the sequence, a tile at the midpoint, and late tiles that few
causal rows see. The gradients are taken on the GPU's own selection;
selection parity at these sizes is the forward workload test's.

The oracle's per-row work runs in threads: a kv tile's sum is split over
(query head, block of query tiles) jobs, each an ``attention_backward`` call
on that head's slice with the keep rows outside its block cleared (a row's
contribution depends only on its own kept tiles, so the partial sums add up
to the whole; they are added in fp64).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
import top_kv_tile_amd as tkt
from oracle.attention_bwd import attention_backward
from parity_util import oracle_workers, say, to_dev
from test_gpu_backward import compare_arrays

pytestmark = pytest.mark.gpu

ROW_BLOCK = 128       # query tiles per oracle job for a kv tile's sum


def _oracle_grads(q, k, v, do, keep, w, rows, kv_tiles):
    """{(b,h,i): dq rows}, {(b,g,j): (dk rows, dv rows)} from the fp64 oracle, in threads."""
    from threadpoolctl import threadpool_limits

    group = w.Hq // w.Hkv
    bsz, hq = w.B, w.Hq

    def plane(b, h):
        return keep[b if keep.shape[0] == bsz else 0, h if keep.shape[1] == hq else 0]

    jobs = []
    for b, h, i in rows:
        jobs.append(("q", b, h, i))
    for b, g, j in kv_tiles:
        for h in range(g * group, (g + 1) * group):
            readers = np.nonzero(plane(b, h)[:, j])[0]
            for i0 in range(0, w.nq, ROW_BLOCK):
                if np.any((readers >= i0) & (readers < i0 + ROW_BLOCK)):
                    jobs.append(("kv", b, h, (g, j, i0)))

    def run(job):
        kind, b, h, x = job
        g = h // group
        sl = (slice(b, b + 1), slice(h, h + 1))
        ks = (slice(b, b + 1), slice(g, g + 1))
        pl = plane(b, h)[None, None].copy()
        if kind == "q":
            dq, _, _ = attention_backward(q[sl], k[ks], v[ks], do[sl], pl, w.block_q, w.block_kv,
                                          w.causal, rows=[(0, 0, x)], kv_tiles=[])
            s = slice(x * w.block_q, min((x + 1) * w.block_q, w.S))
            return kind, (b, h, x), dq[0, 0, s].copy()
        gg, j, i0 = x
        pl[0, 0, :i0] = 0
        pl[0, 0, i0 + ROW_BLOCK:] = 0
        _, dk, dv = attention_backward(q[sl], k[ks], v[ks], do[sl], pl, w.block_q, w.block_kv,
                                       w.causal, rows=[], kv_tiles=[(0, 0, j)])
        s = slice(j * w.block_kv, min((j + 1) * w.block_kv, w.S))
        return kind, (b, gg, j), (dk[0, 0, s].copy(), dv[0, 0, s].copy())

    dq_ref, kv_ref = {}, {}
    for b, g, j in kv_tiles:
        n = min((j + 1) * w.block_kv, w.S) - j * w.block_kv
        kv_ref[(b, g, j)] = (np.zeros((n, w.D)), np.zeros((n, w.D)))
    nthr = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(1), ThreadPoolExecutor(oracle_workers()) as ex:
            for kind, key, val in ex.map(run, jobs):
                if kind == "q":
                    dq_ref[key] = val
                else:
                    kv_ref[key][0][...] += val[0]
                    kv_ref[key][1][...] += val[1]
    finally:
        torch.set_num_threads(nthr)
    return dq_ref, kv_ref


def _stratified_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    idx = np.linspace(0, w.nq - 1, n).round().astype(int)
    rows = {(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(i)) for i in idx}
    return sorted(rows | {(0, 0, 0), (w.B - 1, w.Hq - 1, w.nq - 1)})


def _most_read(keep, w, g, lo, hi):
    """The kv tile in [lo, hi) that the most (query head, query tile) rows of group g keep."""
    group = w.Hq // w.Hkv
    heads = [0] if keep.shape[1] == 1 else list(range(g * group, (g + 1) * group))
    counts = keep[0][heads][:, :, lo:hi].astype(np.int64).sum(axis=(0, 1))
    return lo + int(np.argmax(counts))


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,n_rows", [
    ("gqa_causal_bf16_s16k", 32),
    ("long_causal_gqa_bf16_s128k", 48),
])
def test_backward_workload(name, n_rows):
    w = synth.workload(name)
    say(f"[{name}] generating inputs")
    inp = synth.make_inputs(w)
    g = torch.Generator().manual_seed(4242)
    do = torch.empty(inp.q.shape, dtype=inp.q.dtype)
    for b in range(w.B):                        # per head, to bound host memory
        for h in range(w.Hq):
            do[b, h] = torch.randn(w.S, w.D, generator=g).to(inp.q.dtype)
    qd, kd, vd, dod = (to_dev(t) for t in (inp.q, inp.k, inp.v, do))
    spec = tkt.SparseSpec(budget=w.budget, block_q=w.block_q, block_kv=w.block_kv, head_shared=w.head_shared)
    say(f"[{name}] GPU select, forward, backward")
    sel = tkt.nsa_select(qd, kd, spec, inp.pins, inp.drops)
    out, lse = tkt.nsa_block_sparse_attn(qd, kd, vd, sel, w.causal)
    dq, dk, dv = tkt.nsa_block_sparse_attn_bwd(qd, kd, vd, out, lse, dod, sel, w.causal)
    torch.cuda.synchronize()
    keep = sel.keep.cpu().numpy()
    for name_, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{name}: {name_} has non-finite values"
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    del qd, kd, vd, dod, out, lse, sel
    rows = _stratified_rows(w, n_rows, seed=11)
    mid = w.nk // 2
    tiles = sorted({
        (0, 0, 0),                                               # sink / first tile
        (0, 3, _most_read(keep, w, 3, w.nk * 3 // 8, w.nk * 5 // 8)),  # most-read middle tile
        (0, 5 % w.Hkv, mid),                                     # midpoint
        (w.B - 1, w.Hkv - 1, w.nk - 1),                          # last tile
        (0, 7 % w.Hkv, w.nk - 8),                                # late
    })
    say(f"[{name}] oracle on {len(rows)} query tiles and kv tiles {tiles}")
    dq_ref, kv_ref = _oracle_grads(inp.q, inp.k, inp.v, do, keep, w, rows, tiles)

    def gather(t, keys, block):
        return np.concatenate([t[b, h, i * block:min((i + 1) * block, w.S)].to(torch.float64).numpy()
                               for b, h, i in keys])

    rep = {"dq": compare_arrays("dq", gather(dq, rows, w.block_q),
                                np.concatenate([dq_ref[r] for r in rows]), w.dtype, name)}
    for j, t in ((0, dk), (1, dv)):
        per_tile = {}
        for key in tiles:
            per_tile[key] = compare_arrays(("dk", "dv")[j], gather(t, [key], w.block_kv), kv_ref[key][j],
                                           w.dtype, f"{name} tile {key}")
        rep[("dk", "dv")[j]] = per_tile
    say(f"[{name}] {rep}")
