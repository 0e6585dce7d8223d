"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (fixed by the target of this path):
  * keep flags: bit-exact, except on rows the oracle flags as near ties
    (k-th and (k+1)-th candidate scores within 1e-5 relative), where the GPU
    keep must still be a valid selection (must kept, drops absent, exact count);
  * attention output: fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 1e-3;
  * LSE: max-abs 1e-3 (natural log).
Attention is always compared against the oracle run on the GPU's own keep flags.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import top_kv_tile_amd as tkt

TOL = {"f32": dict(max_abs=1e-4, mean_abs=1e-4), "bf16": dict(max_abs=2e-2, mean_abs=1e-3)}
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: torch.Tensor) -> torch.Tensor:
    return x.to("cuda:0").contiguous()


def check_selection(sel_gpu, ref, where=""):
    """Compare GPU keep / CSR with the oracle dict; returns the GPU keep (numpy int8)."""
    keep = sel_gpu.keep.cpu().numpy()
    row_ptr = sel_gpu.row_ptr.cpu().numpy().astype(np.int64)
    col_idx = sel_gpu.col_idx.cpu().numpy().astype(np.int64)
    assert keep.shape == ref["keep"].shape, (where, keep.shape, ref["keep"].shape)
    assert np.array_equal(row_ptr, ref["row_ptr"]), f"{where}: row_ptr differs"
    # CSR consistent with keep: ascending, in range, same rows
    flat = keep.reshape(-1, keep.shape[-1]) != 0
    assert col_idx.size == row_ptr[-1]
    assert np.all((col_idx >= 0) & (col_idx < keep.shape[-1]))
    r_ptr, r_col = oracle.keep_to_csr(keep)
    assert np.array_equal(r_ptr, row_ptr) and np.array_equal(r_col, col_idx), f"{where}: CSR != keep"
    near = ref["near_tie"].reshape(-1)
    ok_rows = ~near
    gk = flat
    rk = ref["keep"].reshape(-1, keep.shape[-1]) != 0
    mism = np.nonzero(np.any(gk != rk, axis=1) & ok_rows)[0]
    if mism.size:
        r = mism[0]
        s = ref["scores"].reshape(-1, keep.shape[-1])[r]
        raise AssertionError(f"{where}: {mism.size} unflagged rows differ, first row {r}: "
                             f"gpu-only {np.nonzero(gk[r] & ~rk[r])[0][:8]}, "
                             f"oracle-only {np.nonzero(rk[r] & ~gk[r])[0][:8]}, "
                             f"score range {s.min():.4g}..{s.max():.4g}")
    # flagged rows: still a valid selection
    must = ref["must"].reshape(-1, keep.shape[-1])
    forb = ref["forbidden"].reshape(-1, keep.shape[-1])
    assert np.all(gk[must & ~forb]) and not np.any(gk & forb)
    want = (must & ~forb).sum(1) + np.minimum(ref["k"].reshape(-1), ref["c"].reshape(-1))
    assert np.array_equal(gk.sum(1), want)
    return keep, int(near.sum())


def check_attention(out, lse, ref_o, ref_l, dtype: str, rows=None, block_q=None, where="",
                    relative=False):
    """Compare GPU (out, lse) with oracle fp64 arrays, on all rows or (b, h, i) tiles.

    relative=True divides each output error by max(1, |reference|): for stress
    inputs far from N(0, 1) whose outputs reach magnitudes where one bf16 ulp
    alone exceeds the absolute bound."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        sl_o, sl_l, ro, rl = [], [], [], []
        for b, h, i in rows:
            s = slice(i * block_q, min((i + 1) * block_q, o.shape[2]))
            sl_o.append(o[b, h, s]); ro.append(ref_o[b, h, s])
            sl_l.append(l[b, h, s]); rl.append(ref_l[b, h, s])
        o, ref_o = np.concatenate(sl_o), np.concatenate(ro)
        l, ref_l = np.concatenate(sl_l), np.concatenate(rl)
    tol = TOL[dtype]
    err = np.abs(o - ref_o)
    if relative:
        err = err / np.maximum(1.0, np.abs(ref_o))
    assert np.all(np.isfinite(o)), f"{where}: non-finite output"
    assert err.max() <= tol["max_abs"], f"{where}: max-abs {err.max():.3g} > {tol['max_abs']}"
    assert err.mean() <= tol["mean_abs"], f"{where}: mean-abs {err.mean():.3g} > {tol['mean_abs']}"
    both_inf = np.isneginf(l) & np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), f"{where}: -inf LSE rows differ"
    lerr = np.abs(np.where(both_inf, 0.0, l) - np.where(both_inf, 0.0, ref_l))
    assert lerr.max() <= LSE_TOL, f"{where}: LSE max-abs {lerr.max():.3g}"
    return float(err.max()), float(err.mean()), float(lerr.max())


def run_case(q, k, v, spec: tkt.SparseSpec, causal: bool, pins=None, drops=None, rows=None,
             where="", relative=False):
    """Full path on the GPU vs the oracle. Returns a small report dict."""
    dtype = "bf16" if q.dtype == torch.bfloat16 else "f32"
    ref = oracle.select_blocks(q, k, spec.budget, spec.block_q, spec.block_kv, spec.head_shared,
                               spec.force, pins, drops)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sel = tkt.nsa_select(qd, kd, spec, pins, drops)
    torch.cuda.synchronize()
    if ref is None:
        assert sel is None, f"{where}: oracle says dense, GPU returned a selection"
        keep = None
        nflag = 0
    else:
        assert sel is not None, f"{where}: GPU returned dense, oracle has a selection"
        keep, nflag = check_selection(sel, ref, where)
    out, lse = tkt.nsa_block_sparse_attn(qd, kd, vd, sel, causal)
    torch.cuda.synchronize()
    bq = spec.block_q if sel is not None else 128
    bkv = spec.block_kv if sel is not None else 64
    ref_o, ref_l = oracle.attention(q, k, v, keep, bq, bkv, causal, rows=rows)
    errs = check_attention(out, lse, ref_o, ref_l, dtype, rows=rows, block_q=bq, where=where,
                           relative=relative)
    return dict(near_tie_rows=nflag, max_abs=errs[0], mean_abs=errs[1], lse_max=errs[2])
