"""Oracle for the gradients of block-sparse attention, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages make the selected attention trainable only by implication (the NSA
discussion "todo" lists a backward kernel among the open items; the selection
page's keep flags fix which logits exist). What is computed here is the exact
derivative of the forward definition in ``oracle.attention``:

    l_tu = D**-0.5 q_t . k_u           for visible (t, u)
    P_tu = exp(l_tu - LSE_t)
    O_t  = sum_u P_tu v_u

For an upstream gradient dO (same shape as O), with g = h // (Hq / Hkv):

    dV[g, u] += sum_t P_tu dO_t
    dP_tu     = dO_t . v_u
    Delta_t   = sum_u P_tu dP_tu        (equals dO_t . O_t)
    dS_tu     = P_tu (dP_tu - Delta_t)
    dQ_t      = D**-0.5 sum_u dS_tu k_u
    dK[g, u] += D**-0.5 sum_t dS_tu q_t

Visibility is the forward's (kept tile pair, and u <= t under ``causal``).
A query with no visible key contributes nothing. Gradients of the heads of
one GQA group add into their shared kv head.
"""
from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["attention_backward"]


def _row_grads(qt, kk, vv, dot, causal, q_pos, k_pos, scale):
    """fp64 gradients for the query rows qt over their visible keys kk/vv.

    Returns (dq rows, dk rows for kk, dv rows for kk)."""
    nqr, d = qt.shape
    if kk.shape[0] == 0:
        return np.zeros((nqr, d)), np.zeros((0, d)), np.zeros((0, d))
    logits = (qt @ kk.T) * scale
    vis = np.ones(logits.shape, bool)
    if causal:
        vis = k_pos[None, :] <= q_pos[:, None]
    logits = np.where(vis, logits, -np.inf)
    mx = logits.max(axis=1)
    empty = ~np.isfinite(mx)
    mx = np.where(empty, 0.0, mx)
    w = np.where(vis, np.exp(logits - mx[:, None]), 0.0)
    tot = w.sum(axis=1)
    p = w / np.where(empty, 1.0, tot)[:, None]          # rows of empty queries are all zero
    dv = p.T @ dot
    dp = dot @ vv.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = (ds @ kk) * scale
    dk = (ds.T @ qt) * scale
    return dq, dk, dv


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, do: torch.Tensor,
                       keep, block_q: int, block_kv: int, causal: bool, rows=None, kv_tiles=None):
    """Gradients (dQ, dK, dV) of block-sparse attention, fp64 numpy.

    q, do: (B, Hq, S, D); k, v: (B, Hkv, S, D) CPU tensors (fp32 or bf16).
    keep: int8/bool (B', H', NQ, NK) with B' in {1, B}, H' in {1, Hq}, or None
    for dense (all tiles kept).

    By default every output is complete. For large inputs a subset can be
    asked for: ``rows`` lists (b, h, i) query tiles whose dQ rows are wanted,
    ``kv_tiles`` lists (b, g, j) kv tiles whose dK/dV rows are wanted; the
    outputs not asked for stay NaN. A kv tile's gradient is the sum over every
    (query head of group g, query tile) row that keeps it, so each such row is
    evaluated in full.
    """
    bsz, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    if causal and seq_q != seq_kv:
        raise ValueError("causal attention needs seq_q == seq_kv")
    nq = -(-seq_q // block_q)
    nk = -(-seq_kv // block_kv)
    if keep is None:
        keep = np.ones((1, 1, nq, nk), np.int8)
    keep = np.asarray(keep) != 0
    sel_heads = keep.shape[1]
    if hq % hkv != 0 or sel_heads not in (1, hq):
        raise ValueError("need Hq % Hkv == 0 and selection heads in {1, Hq}")
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)

    def tiles_of(b, h, i):
        return np.nonzero(keep[b if keep.shape[0] == bsz else 0, h if sel_heads == hq else 0, i])[0]

    full = rows is None and kv_tiles is None
    if full:
        rows = [(b, h, i) for b in range(bsz) for h in range(hq) for i in range(nq)]
        work = rows
    else:
        rows = list(rows or [])
        want = set(kv_tiles or [])
        work = set(rows)
        for b, g, j in want:
            for h in range(g * group, (g + 1) * group):
                for i in range(nq):
                    # under causal, a query tile that ends before the kv tile starts
                    # adds exactly zero to it and is not evaluated
                    if causal and j * block_kv > min((i + 1) * block_q, seq_q) - 1:
                        continue
                    if keep[b if keep.shape[0] == bsz else 0, h if sel_heads == hq else 0, i, j]:
                        work.add((b, h, i))
        work = sorted(work)
    dq = np.full((bsz, hq, seq_q, d), np.nan)
    dk = np.zeros((bsz, hkv, seq_kv, d))
    dv = np.zeros((bsz, hkv, seq_kv, d))
    dq_rows = set(rows)
    for b, h, i in work:
        g = h // group
        tiles = tiles_of(b, h, i)
        t0, t1 = i * block_q, min((i + 1) * block_q, seq_q)
        pos = [np.arange(j * block_kv, min((j + 1) * block_kv, seq_kv)) for j in tiles]
        k_pos = np.concatenate(pos) if pos else np.zeros(0, np.int64)
        qt = q[b, h, t0:t1].to(torch.float64).numpy()
        dot = do[b, h, t0:t1].to(torch.float64).numpy()
        kk = k[b, g, k_pos].to(torch.float64).numpy()
        vv = v[b, g, k_pos].to(torch.float64).numpy()
        gq, gk, gv = _row_grads(qt, kk, vv, dot, causal, np.arange(t0, t1), k_pos, scale)
        if (b, h, i) in dq_rows:
            dq[b, h, t0:t1] = gq
        dk[b, g, k_pos] += gk                 # k_pos has no repeats within a row
        dv[b, g, k_pos] += gv
    if not full:
        mask = np.zeros((bsz, hkv, seq_kv), bool)
        for b, g, j in kv_tiles or []:
            mask[b, g, j * block_kv:min((j + 1) * block_kv, seq_kv)] = True
        dk[~mask] = np.nan
        dv[~mask] = np.nan
    return dq, dk, dv
