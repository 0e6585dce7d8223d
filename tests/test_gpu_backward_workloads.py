"""GPU parity of the attention gradients at full workload sizes, in the launch
configuration the bench times.

The oracle computes sampled outputs one by one: dQ for seeded (batch, head,
query-tile) rows, and dK / dV for seeded kv tiles, each summed over every query
tile of the GQA group that keeps it. On the 128k workload the sampled kv tiles
sit late in the sequence, where causality leaves few query tiles that see them
(the sink tile 0 is seen by all 8192 rows of its kv head and is covered by the
small cases). The gradients are taken on the GPU's own selection; selection
parity at these sizes is the forward workload test's.
"""
import numpy as np
import pytest
import torch

import synth
import top_kv_tile_amd as tkt
from oracle.attention_bwd import attention_backward
from parity_util import say, to_dev
from test_gpu_backward import _compare

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n_rows,tiles", [
    ("gqa_causal_bf16_s16k", 24, [(0, 0, 255), (1, 3, 200), (0, 7, 129), (1, 5, 40)]),
    ("long_causal_gqa_bf16_s128k", 16, [(0, 0, 2047), (0, 3, 2020), (0, 5, 1990), (0, 7, 2040)]),
])
def test_backward_workload(name, n_rows, tiles):
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
    del qd, kd, vd, dod, out, lse, sel
    rng = np.random.default_rng(11)
    rows = sorted({(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.nq)))
                   for _ in range(n_rows)} | {(0, 0, 0), (w.B - 1, w.Hq - 1, w.nq - 1)})
    say(f"[{name}] oracle on {len(rows)} query tiles and kv tiles {tiles}")
    rq, rk, rv = attention_backward(inp.q, inp.k, inp.v, do, keep, w.block_q, w.block_kv, w.causal,
                                    rows=rows, kv_tiles=tiles)
    rep = {"dq": _compare("dq", dq, rq, w.dtype, ~np.isnan(rq), name),
           "dk": _compare("dk", dk, rk, w.dtype, ~np.isnan(rk), name),
           "dv": _compare("dv", dv, rv, w.dtype, ~np.isnan(rv), name)}
    say(f"[{name}] {rep}")
