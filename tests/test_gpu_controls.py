"""GPU parity of the controls and plan reuse: the radial band (device keep and
CSR against the oracle, then attention and its gradients over that band with one
selection broadcast to every batch entry), planned selection against
nsa_select, the plan cache of nsa_select keyed on the mask contents, and the
host-side density."""
import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from oracle.attention_bwd import attention_backward
from parity_util import check_attention, check_selection, say, to_dev
from test_gpu_backward import _compare

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, S, D, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, h, S, D, generator=g).to(dtype) for h in (Hq, Hkv, Hkv, Hq)]


@pytest.mark.parametrize("S,bq,bkv,dens,causal", [(1000, 128, 64, 0.15, True), (2048, 64, 64, 0.3, False),
                                                  (777, 128, 64, 0.5, True)])
def test_radial_band_attention_and_gradients(S, bq, bkv, dens, causal):
    say(f"radial S={S} bq={bq} bkv={bkv} density={dens} causal={causal}")
    spec = tkt.SparseSpec(block_q=bq, block_kv=bkv)
    sel = tkt.nsa_radial_blocks(S, S, dens, spec)
    torch.cuda.synchronize()
    ref_keep = oracle.radial_blocks(S, S, dens, bq, bkv)
    keep = sel.keep.cpu().numpy()
    assert np.array_equal(keep, ref_keep)
    r_ptr, r_col = oracle.keep_to_csr(ref_keep)
    assert np.array_equal(sel.row_ptr.cpu().numpy(), r_ptr)
    assert np.array_equal(sel.col_idx.cpu().numpy(), r_col)
    assert sel.density() == oracle.density(ref_keep)
    q, k, v, do = _inputs(2, 4, 2, S, 128, seed=S + bq)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = tkt.nsa_block_sparse_attn(qd, kd, vd, sel, causal)   # one band for both batch entries
    ref_o, ref_l = oracle.attention(q, k, v, ref_keep, bq, bkv, causal)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="radial")
    dq, dk, dv = tkt.nsa_block_sparse_attn_bwd(qd, kd, vd, out, lse, dod, sel, causal)
    rq, rk, rv = attention_backward(q, k, v, do, ref_keep, bq, bkv, causal)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _compare(name, got, ref, "bf16", where="radial")


def test_planned_selection_equals_select():
    say("planned selection")
    B, Hq, Hkv, S, D = 2, 4, 2, 1024, 128
    nq, nk = 8, 16
    rng = np.random.default_rng(12)
    pins = (rng.random((B, 1, nq, nk)) < 0.1).astype(np.int8)
    drops = (rng.random((1, Hq, nq, nk)) < 0.1).astype(np.int8)
    spec = tkt.SparseSpec(budget=0.3)
    q0, k0, _, _ = _inputs(B, Hq, Hkv, S, D, seed=1)
    plan = tkt.nsa_plan_create(to_dev(q0), to_dev(k0), spec, pins, drops)
    img = plan.upload(torch.device("cuda:0"))  # the plan's device image, uploaded once
    for seed in (2, 3, 4):  # same shapes, new values: the plan is reused
        q, k, _, _ = _inputs(B, Hq, Hkv, S, D, seed=seed)
        qd, kd = to_dev(q), to_dev(k)
        a = tkt.nsa_select(qd, kd, spec, pins, drops)
        b = tkt.nsa_select_planned(plan, qd, kd)               # image uploaded by the call
        c = tkt.nsa_select_planned(plan, qd, kd, plan_dev=img)  # image from the caller's buffer
        torch.cuda.synchronize()
        for x in (b, c):
            assert torch.equal(a.keep, x.keep) and torch.equal(a.row_ptr, x.row_ptr)
            assert torch.equal(a.col_idx, x.col_idx)
        assert abs(b.density() - float(b.keep.float().mean().item())) < 1e-12
    dense_plan = tkt.nsa_plan_create(to_dev(q0), to_dev(k0), tkt.SparseSpec(budget=1.0))
    assert tkt.nsa_select_planned(dense_plan, to_dev(q0), to_dev(k0)) is None


def test_select_plan_cache_keys_on_masks():
    """nsa_select caches its plan. A call whose drops differ from the previous
    call's in one candidate tile (same shapes, spec and pins) gets the plan of
    its own masks, and the first mask set still finds its own: every selection
    matches the oracle for the masks it was given."""
    say("plan cache keyed on masks")
    B, Hq, Hkv, S, D, bq, bkv, budget = 1, 4, 2, 2048, 128, 128, 64, 0.25
    nq, nk = S // bq, S // bkv
    rng = np.random.default_rng(5)
    pins = np.zeros((1, 1, nq, nk), np.int8)
    pins[..., 0] = 1
    drops = (rng.random((1, Hq, nq, nk)) < 0.05).astype(np.int8)
    plan = oracle.selection_plan(nq, nk, bq, bkv, budget, B, Hq, pins, drops)
    flip = None
    for h in range(Hq):
        for i in range(nq):
            c = int(plan["c"][0, h, i])
            if c > 1 and int(oracle.keep_per_row(np.array([c - 1]), budget)[0]) != int(plan["k"][0, h, i]):
                flip = (h, i, int(np.nonzero(plan["candidates"][0, h, i])[0][0]))
                break
        if flip:
            break
    assert flip is not None
    drops2 = drops.copy()
    drops2[0, flip[0], flip[1], flip[2]] = 1
    q, k, _, _ = _inputs(B, Hq, Hkv, S, D, seed=9)
    qd, kd = to_dev(q), to_dev(k)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv)
    tkt.nsa_plan_cache_clear()
    nnz = []
    for d in (drops, drops2, drops):
        sel = tkt.nsa_select(qd, kd, spec, pins, d)
        ref = oracle.select_blocks(q, k, budget, bq, bkv, False, False, pins, d)
        check_selection(sel, ref, "cached plan")
        nnz.append(int(sel.row_ptr[-1].item()))
    assert nnz[0] != nnz[1] and nnz[0] == nnz[2]
    hits, misses, _ = tkt.nsa_plan_cache_stats()
    assert misses == 2 and hits == 4  # nsa_select_sizes and nsa_select look up once each per call
