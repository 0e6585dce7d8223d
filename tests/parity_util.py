"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (fixed by the target of this path):
  * keep flags: bit-exact, except on rows the oracle flags as near ties
    (k-th and (k+1)-th candidate scores within 1e-5 relative), where the GPU
    keep must still be a valid selection (must kept, drops absent, exact count)
    that differs from the oracle's only by trading candidates inside the
    near-tie band of the row's k-th score;
  * attention output: fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 1e-3;
  * LSE: max-abs 1e-3 (natural log).
Attention is always compared against the oracle run on the GPU's own keep flags.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

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
    # every row: must kept, drops absent, exact count
    must = ref["must"].reshape(-1, keep.shape[-1])
    forb = ref["forbidden"].reshape(-1, keep.shape[-1])
    assert np.all(gk[must & ~forb]) and not np.any(gk & forb)
    want = (must & ~forb).sum(1) + np.minimum(ref["k"].reshape(-1), ref["c"].reshape(-1))
    assert np.array_equal(gk.sum(1), want)
    check_near_tie_rows(gk, rk, ref, where)
    return keep, int(near.sum())


def check_near_tie_rows(gk, rk, ref, where=""):
    """On flagged rows the GPU may differ from the oracle only by exchanging
    candidates whose oracle scores tie with the row's k-th candidate score.

    selector.py, ``select_blocks``: the picks are the first k_r candidates of a
    stable descending order, so the only freedom a different fp32 summation
    order has is at the cut. Every tile in the symmetric difference must be a
    candidate, the two sides must trade equal numbers of tiles, and each traded
    tile's oracle score s_j must lie in the near-tie band of the k-th score
    s_(k): |s_j - s_(k)| <= NEAR_TIE_REL * max(|s_j|, |s_(k)|).
    Returns the number of flagged rows that differ from the oracle."""
    nk = gk.shape[-1]
    near = ref["near_tie"].reshape(-1)
    cand = (~ref["must"] & ~ref["forbidden"]).reshape(-1, nk)
    scores = ref["scores"].reshape(-1, nk).astype(np.float64)
    kr = ref["k"].reshape(-1)
    differing = 0
    for r in np.nonzero(near)[0]:
        g_only = np.nonzero(gk[r] & ~rk[r])[0]
        o_only = np.nonzero(rk[r] & ~gk[r])[0]
        if g_only.size == 0 and o_only.size == 0:
            continue
        differing += 1
        assert g_only.size == o_only.size, f"{where}: row {r} trades {g_only.size} for {o_only.size} tiles"
        assert np.all(cand[r, g_only]) and np.all(cand[r, o_only]), f"{where}: row {r} trades a non-candidate"
        cs = np.sort(scores[r, cand[r]])[::-1]
        s_k = cs[kr[r] - 1]
        for j in np.concatenate([g_only, o_only]):
            band = oracle.NEAR_TIE_REL * max(abs(scores[r, j]), abs(s_k))
            assert abs(scores[r, j] - s_k) <= band, (
                f"{where}: row {r} tile {j} score {scores[r, j]!r} outside the tie band of "
                f"s_(k) = {s_k!r}")
    return differing


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


def oracle_workers() -> int:
    """Threads for the oracle's per-row work: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_attention_rows(q, k, v, keep, block_q, block_kv, causal, rows, chunk=32):
    """fp64 oracle attention of the listed (b, h, i) query tiles, in parallel threads.

    Each job runs ``oracle.attention`` on one query head's slice: q[b, h], the
    kv head k[b, h // (Hq/Hkv)] / v[b, ...] it reads, and its selection plane
    keep[b or 0, h or 0]. That is the oracle's own problem restricted to one
    head; the head mapping is the one ``oracle.attention`` applies (pinned
    against SDPA for GQA in the oracle tests, and exercised on full tensors by
    the small parity cases). BLAS is held to one thread per job so the
    threads do not oversubscribe the cores.
    Returns {(b, h, i): (O fp64 (rows of the tile, D), LSE fp64)}."""
    from threadpoolctl import threadpool_limits

    bsz, hq = q.shape[0], q.shape[1]
    group = hq // k.shape[1]
    keep = np.asarray(keep)
    by_head = {}
    for b, h, i in rows:
        by_head.setdefault((b, h), []).append(i)
    jobs = []
    for (b, h), tiles in sorted(by_head.items()):
        tiles = sorted(tiles)
        for c in range(0, len(tiles), chunk):
            jobs.append((b, h, tiles[c:c + chunk]))

    def run(job):
        b, h, tiles = job
        g = h // group
        kb = b if keep.shape[0] == bsz else 0
        hs = h if keep.shape[1] == hq else 0
        o, l = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                keep[kb:kb + 1, hs:hs + 1], block_q, block_kv, causal,
                                rows=[(0, 0, i) for i in tiles])
        seq = q.shape[2]
        res = {}
        for i in tiles:
            s = slice(i * block_q, min((i + 1) * block_q, seq))
            res[(b, h, i)] = (o[0, 0, s].copy(), l[0, 0, s].copy())
        return res

    out = {}
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(1), ThreadPoolExecutor(oracle_workers()) as ex:
            for res in ex.map(run, jobs):
                out.update(res)
    finally:
        torch.set_num_threads(torch_threads)
    return out


def check_attention_rows(out, lse, refs, dtype: str, block_q: int, where=""):
    """Compare the GPU (out, lse) with oracle rows from ``oracle_attention_rows``.

    Same bounds as ``check_attention`` over the union of the listed rows: output
    max-abs and mean-abs, LSE max-abs, -inf rows identical."""
    o_cpu = out.cpu()
    l_cpu = lse.cpu()
    seq = o_cpu.shape[2]
    tol = TOL[dtype]
    emax, esum, n, lmax = 0.0, 0.0, 0, 0.0
    worst = None
    for (b, h, i), (ro, rl) in refs.items():
        s = slice(i * block_q, min((i + 1) * block_q, seq))
        o = o_cpu[b, h, s].to(torch.float64).numpy()
        l = l_cpu[b, h, s].to(torch.float64).numpy()
        assert np.all(np.isfinite(o)), f"{where}: non-finite output in row {(b, h, i)}"
        err = np.abs(o - ro)
        if err.max() > emax:
            emax, worst = float(err.max()), (b, h, i)
        esum += float(err.sum())
        n += err.size
        assert np.array_equal(np.isneginf(l), np.isneginf(rl)), f"{where}: -inf LSE differs in row {(b, h, i)}"
        both = np.isneginf(l)
        lmax = max(lmax, float(np.abs(np.where(both, 0.0, l) - np.where(both, 0.0, rl)).max()))
    mean = esum / max(n, 1)
    assert emax <= tol["max_abs"], f"{where}: max-abs {emax:.3g} > {tol['max_abs']} (row {worst})"
    assert mean <= tol["mean_abs"], f"{where}: mean-abs {mean:.3g} > {tol['mean_abs']}"
    assert lmax <= LSE_TOL, f"{where}: LSE max-abs {lmax:.3g}"
    return emax, mean, lmax
