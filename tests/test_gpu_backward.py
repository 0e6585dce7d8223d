"""GPU parity of the attention gradients: the HIP path (through the C ABI) against
the fp64 gradient oracle, on the GPU's own selection.

Tolerances (derived from the arithmetic; each error is taken relative to the
largest magnitude of the reference tensor it belongs to):
  * fp32 inputs: max 1e-4 and mean 1e-4 (fp32 accumulation, fp32 P and dS);
  * bf16 inputs: max 2e-2 and mean 5e-3 of the mean magnitude. The kernels
    round P and dS to bf16 for the matrix cores (2^-9 relative each), take
    Delta from the bf16 forward output, and round the results to bf16. The
    final rounding alone gives a mean relative error near 2^-9 * 0.7 ~ 1.4e-3
    (round-to-nearest on an 8-bit significand); the bound leaves about 3.5x
    that for the P and dS roundings, whose sums have random signs.
Outputs are prefilled with NaN, so every element must be written.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from oracle.attention_bwd import attention_backward
from parity_util import check_selection, say, to_dev

pytestmark = pytest.mark.gpu

GRAD_TOL = {"f32": dict(max_rel=1e-4, mean_rel=1e-4), "bf16": dict(max_rel=2e-2, mean_rel=5e-3)}


def _inputs(B, Hq, Hkv, S, D, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, S, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, S, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, S, D, generator=g).to(dtype)
    do = torch.randn(B, Hq, S, D, generator=g).to(dtype)
    return q, k, v, do


def _compare(name, got, ref, dtype, mask=None, where=""):
    g = got.float().cpu().numpy().astype(np.float64)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    return compare_arrays(name, g, ref, dtype, where)


def compare_arrays(name, g, ref, dtype, where=""):
    """Gradient bounds of this file on fp64 numpy arrays (GPU values, oracle values)."""
    assert np.all(np.isfinite(g)), f"{where}: {name} has non-finite values (unwritten?)"
    assert np.all(np.isfinite(ref))
    tol = GRAD_TOL[dtype]
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(g - ref)
    max_rel = err.max() / scale
    mean_rel = err.mean() / max(np.abs(ref).mean(), 1e-30)
    assert max_rel <= tol["max_rel"], f"{where}: {name} max error {max_rel:.3g} of max |ref| > {tol['max_rel']}"
    assert mean_rel <= tol["mean_rel"], f"{where}: {name} mean error {mean_rel:.3g} of mean |ref|"
    return max_rel, mean_rel


def run_bwd_case(q, k, v, do, spec, causal, pins=None, drops=None, rows=None, kv_tiles=None, where=""):
    """select -> forward -> backward on the GPU; gradients vs the oracle on the GPU's keep."""
    dtype = "bf16" if q.dtype == torch.bfloat16 else "f32"
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    sel = None if spec is None else tkt.nsa_select(qd, kd, spec, pins, drops)
    if spec is not None and sel is not None:
        ref = oracle.select_blocks(q, k, spec.budget, spec.block_q, spec.block_kv, spec.head_shared,
                                   spec.force, pins, drops)
        keep, _ = check_selection(sel, ref, where)
        bq, bkv = spec.block_q, spec.block_kv
    else:
        keep, bq, bkv = None, 128, 64
    out, lse = tkt.nsa_block_sparse_attn(qd, kd, vd, sel, causal)
    nan = float("nan")
    dq = torch.full_like(qd, nan)
    dk = torch.full_like(kd, nan)
    dv = torch.full_like(vd, nan)
    tkt.nsa_block_sparse_attn_bwd(qd, kd, vd, out, lse, dod, sel, causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rq, rk, rv = attention_backward(q, k, v, do, keep, bq, bkv, causal, rows=rows, kv_tiles=kv_tiles)
    mq = None if rows is None else ~np.isnan(rq)
    mk = None if kv_tiles is None else ~np.isnan(rk)
    rep = {}
    if rows is None or rows:
        rep["dq"] = _compare("dq", dq, rq, dtype, mq, where)
    if kv_tiles is None or kv_tiles:
        rep["dk"] = _compare("dk", dk, rk, dtype, mk, where)
        rep["dv"] = _compare("dv", dv, rv, dtype, mk, where)
    # every element written, also where the oracle was not asked
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{where}: {name} not fully written"
    return rep


CASES = [
    # name, B, Hq, Hkv, S, D, bq, bkv, budget, shared, causal, dtype
    ("f32_tiny_causal", 1, 2, 2, 512, 64, 64, 32, 0.30, False, True, torch.float32),
    ("bf16_gqa_causal_ragged", 2, 4, 2, 1000, 128, 128, 64, 0.30, False, True, torch.bfloat16),
    ("bf16_shared_noncausal_ragged", 1, 4, 4, 777, 128, 128, 64, 0.25, True, False, torch.bfloat16),
    ("bf16_d64_bq64_gqa8", 1, 8, 1, 2048, 64, 64, 64, 0.20, False, True, torch.bfloat16),
    ("bf16_bq32", 1, 2, 2, 640, 128, 32, 64, 0.40, False, True, torch.bfloat16),
    ("bf16_bq96_ragged", 1, 2, 1, 1000, 128, 96, 64, 0.30, False, True, torch.bfloat16),
    ("bf16_general_kernel_bkv32", 1, 2, 1, 700, 64, 64, 32, 0.30, False, True, torch.bfloat16),
    ("f32_d128_noncausal", 1, 2, 2, 600, 128, 128, 64, 0.50, False, False, torch.float32),
    ("bf16_d64_shared_causal", 2, 4, 2, 900, 64, 128, 64, 0.30, True, True, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, B, Hq, Hkv, S, D, bq, bkv, budget, shared, causal, dtype = case
    say(f"bwd case {name}")
    q, k, v, do = _inputs(B, Hq, Hkv, S, D, seed=zlib.crc32(name.encode()) % 10000, dtype=dtype)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv, head_shared=shared)
    rep = run_bwd_case(q, k, v, do, spec, causal, where=name)
    say(f"  {rep}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_dense(causal):
    say(f"bwd dense causal={causal}")
    q, k, v, do = _inputs(1, 4, 2, 1000, 128, seed=12, dtype=torch.bfloat16)
    rep = run_bwd_case(q, k, v, do, None, causal, where="dense")
    say(f"  {rep}")


def test_backward_pins_drops_and_empty_rows():
    """A dropped diagonal makes causal query rows with no visible key: they get
    no gradient and add nothing to dK / dV."""
    say("bwd pins/drops")
    B, Hq, Hkv, S, D, bq, bkv = 2, 4, 2, 1024, 128, 128, 64
    q, k, v, do = _inputs(B, Hq, Hkv, S, D, seed=78, dtype=torch.bfloat16)
    nq, nk = 8, 16
    rng = np.random.default_rng(6)
    pins = (rng.random((B, 1, nq, nk)) < 0.1).astype(np.int8)
    drops = (rng.random((1, Hq, nq, nk)) < 0.1).astype(np.int8)
    drops[0, 1, 3, 6] = 1
    drops[0, 1, 3, 7] = 1
    pins[:, :, 3, :] = 0
    drops[0, 2, 0, 0] = 1                 # query tile 0 of head 2: only its diagonal tiles 0, 1
    drops[0, 2, 0, 1] = 1
    pins[:, :, 0, :] = 0
    spec = tkt.SparseSpec(budget=0.3, block_q=bq, block_kv=bkv)
    rep = run_bwd_case(q, k, v, do, spec, True, pins=pins, drops=drops, where="pins_drops")
    say(f"  {rep}")


def test_backward_growing_logits():
    """Keys whose scale grows along the sequence: P near one on late keys, large dS."""
    say("bwd growing logits")
    B, H, S, D = 1, 2, 2048, 128
    q, k, v, do = _inputs(B, H, H, S, D, seed=32, dtype=torch.float32)
    ramp = (1.0 + torch.arange(S, dtype=torch.float32) / 256.0)[None, None, :, None]
    k = (k * ramp).to(torch.bfloat16)
    q, v, do = q.to(torch.bfloat16), v.to(torch.bfloat16), do.to(torch.bfloat16)
    rep = run_bwd_case(q, k, v, do, tkt.SparseSpec(budget=0.5), True, where="growing")
    say(f"  {rep}")


def test_backward_twice_reuses_workspace():
    """Two calls with one workspace give identical results (the index is rebuilt each call)."""
    say("bwd twice")
    q, k, v, do = (to_dev(t) for t in _inputs(1, 4, 2, 1000, 128, seed=5, dtype=torch.bfloat16))
    spec = tkt.SparseSpec(budget=0.3)
    sel = tkt.nsa_select(q, k, spec)
    out, lse = tkt.nsa_block_sparse_attn(q, k, v, sel, True)
    ws = torch.empty(tkt.nsa_attn_bwd_workspace_size(q, k, sel), dtype=torch.uint8, device=q.device)
    g1 = tkt.nsa_block_sparse_attn_bwd(q, k, v, out, lse, do, sel, True, workspace=ws)
    g2 = tkt.nsa_block_sparse_attn_bwd(q, k, v, out, lse, do, sel, True, workspace=ws)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_empty_sequence():
    say("bwd empty")
    q = torch.zeros(1, 2, 0, 64, device="cuda:0")
    sel = tkt.nsa_select(q, q, tkt.SparseSpec(budget=0.3, force=True))
    out, lse = tkt.nsa_block_sparse_attn(q, q, q, sel, True)
    dq, dk, dv = tkt.nsa_block_sparse_attn_bwd(q, q, q, out, lse, q, sel, True)
    assert dq.numel() == 0 and dk.numel() == 0 and dv.numel() == 0
