"""GPU parity on the five named workloads at their full sizes.

Selection: every row of every workload is compared with the oracle (keep flags
bit-exact outside near-tie rows, CSR identical). Attention: all rows of the
tiny fp32 workload; on the large ones, seeded samples of (batch, head,
query-tile) rows plus every near-tie row, each computed by the oracle one by
one, in the same launch configuration the bench times.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
import top_kv_tile_amd as tkt
from parity_util import check_attention, check_selection, say, to_dev

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _prepared(name):
    w = synth.workload(name)
    say(f"[{name}] generating inputs")
    inp = synth.make_inputs(w)
    say(f"[{name}] oracle selection")
    ref = oracle.select_blocks(inp.q, inp.k, w.budget, w.block_q, w.block_kv, w.head_shared, False,
                               inp.pins, inp.drops)
    return w, inp, ref


def _sample_rows(w, ref, n, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for _ in range(n):
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.nq))))
    rows.add((w.B - 1, w.Hq - 1, w.nq - 1))
    rows.add((0, 0, 0))
    # every near-tie row (its selection head maps to query heads h' or all heads)
    for b, hs, i in zip(*np.nonzero(ref["near_tie"])):
        rows.add((int(b), int(hs) if not w.head_shared else 0, int(i)))
    return sorted(rows)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n_rows", [
    ("tiny_causal_f32", None),
    ("mha_bf16_s8k", 96),
    ("gqa_causal_bf16_s16k", 96),
    ("grid2d_morton_shared_bf16", 96),
    ("long_causal_gqa_bf16_s128k", 192),
])
def test_workload(name, n_rows):
    w, inp, ref = _prepared(name)
    say(f"[{name}] GPU select")
    qd, kd, vd = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    spec = tkt.SparseSpec(budget=w.budget, block_q=w.block_q, block_kv=w.block_kv, head_shared=w.head_shared)
    sel = tkt.nsa_select(qd, kd, spec, inp.pins, inp.drops)
    torch.cuda.synchronize()
    keep, nflag = check_selection(sel, ref, name)
    say(f"[{name}] selection matches (near-tie rows {nflag}, nnz {sel.nnz}); GPU attention")
    out, lse = tkt.nsa_block_sparse_attn(qd, kd, vd, sel, w.causal)
    torch.cuda.synchronize()
    del qd, kd, vd
    rows = None if n_rows is None else _sample_rows(w, ref, n_rows, seed=7)
    say(f"[{name}] oracle attention on {'all' if rows is None else len(rows)} rows")
    ref_o, ref_l = oracle.attention(inp.q, inp.k, inp.v, keep, w.block_q, w.block_kv, w.causal, rows=rows)
    errs = check_attention(out, lse, ref_o, ref_l, w.dtype, rows=rows, block_q=w.block_q, where=name)
    say(f"[{name}] attention max-abs {errs[0]:.3g} mean-abs {errs[1]:.3g} lse {errs[2]:.3g}")
