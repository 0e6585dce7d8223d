"""Stage timing through the C ABI: the selection and gradient calls record their
stages while timing is on, and their results are bit-identical with and without it."""
import numpy as np
import pytest
import torch

import top_kv_tile_amd as tkt
from parity_util import say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed=11, B=1, Hq=8, Hkv=2, S=4096, D=128):
    g = torch.Generator().manual_seed(seed)
    mk = lambda H: torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    return mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)


def test_selection_and_gradient_stages():
    say("stage timing: selection and gradients")
    q, k, v, do = (to_dev(x) for x in _inputs())
    spec = tkt.SparseSpec(budget=0.2, block_q=128, block_kv=64)

    ref_sel = tkt.nsa_select(q, k, spec)
    out, lse = tkt.nsa_block_sparse_attn(q, k, v, ref_sel, True)
    ref_dq, ref_dk, ref_dv = tkt.nsa_block_sparse_attn_bwd(q, k, v, out, lse, do, ref_sel, True)
    torch.cuda.synchronize()

    tkt.nsa_stage_timing_begin()
    sel = tkt.nsa_select(q, k, spec)
    dq, dk, dv = tkt.nsa_block_sparse_attn_bwd(q, k, v, out, lse, do, sel, True)
    recs = tkt.nsa_stage_timing_end()
    names = [n for n, _ in recs]
    say(f"  stages {names}")
    # selection: pooling, then one score and one top-k launch per head chunk
    assert names[:2] == ["pool_q", "pool_k"]
    sel_names = names[:names.index("delta")]
    assert sel_names.count("scores") == sel_names.count("topk") >= 1
    # gradients, in launch order
    assert names[len(sel_names):] == ["delta", "kv_index", "dq", "dkdv"]
    assert all(ms >= 0.0 and np.isfinite(ms) for _, ms in recs)

    for a, b in ((sel.keep, ref_sel.keep), (sel.row_ptr, ref_sel.row_ptr), (sel.col_idx, ref_sel.col_idx),
                 (dq, ref_dq), (dk, ref_dk), (dv, ref_dv)):
        assert torch.equal(a, b)


def test_timing_off_records_nothing():
    q, k, _, _ = (to_dev(x) for x in _inputs(S=1024))
    tkt.nsa_stage_timing_begin()
    assert tkt.nsa_stage_timing_end() == []
    tkt.nsa_select(q, k, tkt.SparseSpec(budget=0.2, block_q=128, block_kv=64))
    torch.cuda.synchronize()
    tkt.nsa_stage_timing_begin()  # a new run drops nothing that was never recorded
    assert tkt.nsa_stage_timing_end() == []
