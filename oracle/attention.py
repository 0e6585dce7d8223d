"""Oracle for block-sparse attention over the kept KV tiles, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

No page prints the attention consumer; what it computes is the plain reading of
the selection page ("automatic/modules/attention/sparse/selector.py",
``BlockSelection``: the keep flags are the geometry every consumer reads) plus
the usual attention conventions, each a reading where the page shows no attention call:

* query head h reads kv head g = h // (Hq / Hkv) and selection head h' = h, or
  0 when the selection is shared by all heads;
* key u is visible to query t iff the tile pair (t // bq, u // bkv) is kept and,
  with ``causal``, u <= t (top-left aligned, seq_q == seq_kv);
* logits l_tu = D**-0.5 * q_t . k_u; LSE_t = ln sum_{visible u} exp(l_tu);
  O_t = sum_{visible u} exp(l_tu - LSE_t) v_u;
* a query with no visible key has O_t = 0 and LSE_t = -inf.

``attention`` evaluates each (b, h, q-tile) row over the gathered keys of its
kept tiles (masked terms contribute exactly zero, so this equals dense masking);
``attention_dense_literal`` builds the S x S mask and is used to check that on
small inputs.
"""
from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["attention", "attention_dense_literal", "visible_key_counts"]


def _row(qt, kk, vv, causal, q_pos, k_pos, scale):
    """fp64 softmax attention of the query rows qt over keys kk/vv (numpy fp64)."""
    nqr = qt.shape[0]
    d = qt.shape[1]
    if kk.shape[0] == 0:
        return np.zeros((nqr, d)), np.full(nqr, -np.inf)
    logits = (qt @ kk.T) * scale
    if causal:
        logits = np.where(k_pos[None, :] <= q_pos[:, None], logits, -np.inf)
    mx = logits.max(axis=1)
    empty = ~np.isfinite(mx)
    mx = np.where(empty, 0.0, mx)
    w = np.exp(logits - mx[:, None])
    tot = w.sum(axis=1)
    lse = np.where(empty, -np.inf, mx + np.log(np.where(empty, 1.0, tot)))
    out = np.where(empty[:, None], 0.0, (w @ vv) / np.where(empty, 1.0, tot)[:, None])
    return out, lse


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep, block_q: int,
              block_kv: int, causal: bool, rows=None, q_offset=None):
    """Block-sparse attention in fp64 over the kept tiles.

    q: (B, Hq, S, D); k, v: (B, Hkv, S, D) CPU tensors (fp32 or bf16).
    keep: int8/bool (B, H', NQ, NK) with H' in {1, Hq}, or None for dense (all tiles).
    rows: optional iterable of (b, h, i) query rows to evaluate (others stay
    NaN in the output); default all rows.
    q_offset (decode reading, not on the pages): query t sits at absolute key
    position q_offset + t, so causal visibility is u <= q_offset + t; seq_q and
    seq_kv may then differ. None keeps the top-left alignment with seq_q == seq_kv.
    Returns (O fp64 (B, Hq, S, D), LSE fp64 (B, Hq, S)) as numpy arrays.
    """
    bsz, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    if causal and seq_q != seq_kv and q_offset is None:
        raise ValueError("causal attention needs seq_q == seq_kv")
    off = 0 if q_offset is None else int(q_offset)
    nq = -(-seq_q // block_q)
    nk = -(-seq_kv // block_kv)
    if keep is None:
        keep = np.ones((1, 1, nq, nk), np.int8)
    keep = np.asarray(keep)
    sel_heads = keep.shape[1]
    if hq % hkv != 0 or sel_heads not in (1, hq):
        raise ValueError("need Hq % Hkv == 0 and selection heads in {1, Hq}")
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out = np.full((bsz, hq, seq_q, d), np.nan)
    lse = np.full((bsz, hq, seq_q), np.nan)
    if rows is None:
        rows = [(b, h, i) for b in range(bsz) for h in range(hq) for i in range(nq)]
    for b, h, i in rows:
        g = h // group
        hs = h if sel_heads == hq else 0
        kb = b if keep.shape[0] == bsz else 0
        tiles = np.nonzero(keep[kb, hs, i])[0]
        t0, t1 = i * block_q, min((i + 1) * block_q, seq_q)
        pos = [np.arange(j * block_kv, min((j + 1) * block_kv, seq_kv)) for j in tiles]
        k_pos = np.concatenate(pos) if pos else np.zeros(0, np.int64)
        qt = q[b, h, t0:t1].to(torch.float64).numpy()
        kk = k[b, g, k_pos].to(torch.float64).numpy()
        vv = v[b, g, k_pos].to(torch.float64).numpy()
        o, l = _row(qt, kk, vv, causal, off + np.arange(t0, t1), k_pos, scale)
        out[b, h, t0:t1] = o
        lse[b, h, t0:t1] = l
    return out, lse


def attention_dense_literal(q, k, v, keep, block_q: int, block_kv: int, causal: bool):
    """Same result as ``attention`` from a literal (S_q x S_kv) token mask.

    Builds visible(t, u) = keep[t // bq, u // bkv] and (not causal or u <= t)
    for every token pair and runs one masked softmax per query head. Only for
    small inputs.
    """
    bsz, hq, seq_q, d = q.shape
    hkv, seq_kv = k.shape[1], k.shape[2]
    nq = -(-seq_q // block_q)
    nk = -(-seq_kv // block_kv)
    if keep is None:
        keep = np.ones((1, 1, nq, nk), np.int8)
    keep = np.asarray(keep) != 0
    group = hq // hkv
    scale = 1.0 / math.sqrt(d)
    tq = np.arange(seq_q) // block_q
    tk = np.arange(seq_kv) // block_kv
    out = np.zeros((bsz, hq, seq_q, d))
    lse = np.zeros((bsz, hq, seq_q))
    for b in range(bsz):
        for h in range(hq):
            g = h // group
            km = keep[b if keep.shape[0] == bsz else 0, h if keep.shape[1] == hq else 0]
            vis = km[tq[:, None], tk[None, :]]
            if causal:
                vis = vis & (np.arange(seq_kv)[None, :] <= np.arange(seq_q)[:, None])
            qq = q[b, h].to(torch.float64).numpy()
            kk = k[b, g].to(torch.float64).numpy()
            vv = v[b, g].to(torch.float64).numpy()
            logits = np.where(vis, (qq @ kk.T) * scale, -np.inf)
            mx = logits.max(axis=1)
            empty = ~np.isfinite(mx)
            mx = np.where(empty, 0.0, mx)
            w = np.exp(logits - mx[:, None])
            tot = w.sum(axis=1)
            lse[b, h] = np.where(empty, -np.inf, mx + np.log(np.where(empty, 1.0, tot)))
            out[b, h] = np.where(empty[:, None], 0.0, (w @ vv) / np.where(empty, 1.0, tot)[:, None])
    return out, lse


def visible_key_counts(keep, block_q: int, block_kv: int, seq_q: int, seq_kv: int, causal: bool):
    """Number of keys each query token sees, (B', H', S_q) int64 (for closed-form checks)."""
    keep = np.asarray(keep) != 0
    tq = np.arange(seq_q) // block_q
    cnt = np.zeros(keep.shape[:2] + (seq_q,), np.int64)
    for b in range(keep.shape[0]):
        for h in range(keep.shape[1]):
            for t in range(seq_q):
                tiles = np.nonzero(keep[b, h, tq[t]])[0]
                n = 0
                for j in tiles:
                    lo, hi = j * block_kv, min((j + 1) * block_kv, seq_kv)
                    if causal:
                        hi = min(hi, t + 1)
                    n += max(0, hi - lo)
                cnt[b, h, t] = n
    return cnt
