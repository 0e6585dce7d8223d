"""Oracle for the selection stage: which KV tiles each query tile keeps.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain CPU code in
numpy / torch-CPU, fp32 where the page computes in fp32.

Everything here follows the page "automatic/modules/attention/sparse/selector.py"
(cited below as *selector.py*), function by function:

* ``block_count``      -- ceil division of a length into blocks.
* ``pool_blocks``      -- fp32 mean of each block of tokens, the tail block
                          averaged over its real length.
* ``diagonal_blocks``  -- tiles whose query and key token ranges intersect.
* ``score_blocks``     -- raw pooled dot product, no scale and no softmax;
                          head-shared means over heads, or GQA repeat of the
                          pooled keys onto the query heads.
* ``selection_plan``   -- must = diagonal OR pins; forbidden = drops;
                          candidates = neither; per-row budget
                          ceil(candidates x budget) in fp32.
* ``select_blocks``    -- dense short circuit, then per row the first
                          ``k_r`` candidates in (score descending, kv index
                          ascending) order, joined with must, minus forbidden.

Readings where the page is silent (the plainest reading the rest of the page supports):
* The per-row budget multiplies an integer count by a Python float, which
  torch promotes to float32: k_r = ceil(fl32(fl32(c_r) * fl32(budget))).
* Drops win over must (the forbidden set is removed last).
* -0.0 and +0.0 compare equal; ties go to the lower kv index.
* Scores must be finite.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "block_count",
    "pool_blocks",
    "diagonal_blocks",
    "head_operands",
    "score_blocks",
    "selection_plan",
    "keep_per_row",
    "select_blocks",
    "keep_to_csr",
    "rank_select",
    "NEAR_TIE_REL",
]

# Relative gap under which the k-th and (k+1)-th candidate scores of a row are
# treated as tied (a GPU whose fp32 sums run in another order may swap them).
NEAR_TIE_REL = 1e-5


def block_count(length: int, block: int) -> int:
    """Number of blocks of ``block`` tokens covering ``length`` tokens (ceil).

    selector.py, ``block_count``.
    """
    return -(-int(length) // int(block))


def pool_blocks(x: torch.Tensor, block: int) -> torch.Tensor:
    """fp32 mean over each block of ``block`` tokens along dim -2.

    selector.py, ``pool_blocks``: the sum runs in fp32 and is divided by the
    number of tokens the block really holds, so the last (tail) block is the
    mean over its own length, with no padding.

    x: (..., S, D) float tensor (fp32 or bf16). Returns (..., ceil(S/block), D) fp32.
    """
    seq = x.shape[-2]
    n = block_count(seq, block)
    out = torch.empty(x.shape[:-2] + (n, x.shape[-1]), dtype=torch.float32)
    for i in range(n):
        lo, hi = i * block, min((i + 1) * block, seq)
        seg = x[..., lo:hi, :].to(torch.float32)
        out[..., i, :] = seg.sum(dim=-2, dtype=torch.float32) / float(hi - lo)
    return out


def diagonal_blocks(nq: int, nk: int, block_q: int, block_kv: int, q_offset: int = 0) -> np.ndarray:
    """Boolean (nq, nk): query tile i and kv tile j cover intersecting token ranges.

    selector.py, ``diagonal_blocks``: tile i spans tokens [i*bq, (i+1)*bq) and
    tile j spans [j*bkv, (j+1)*bkv) (unclipped); the pair is on the diagonal when
    each range starts before the other ends. Keeping these tiles guarantees
    every query row keeps at least one tile.

    ``q_offset`` (decode reading, not on the page): the query tokens sit at
    absolute positions q_offset + t of the key sequence, so tile i spans
    [q_offset + i*bq, q_offset + (i+1)*bq). 0 is the page's alignment.
    """
    i = np.arange(nq, dtype=np.int64)[:, None]
    j = np.arange(nk, dtype=np.int64)[None, :]
    return (q_offset + i * block_q < (j + 1) * block_kv) & (j * block_kv < q_offset + (i + 1) * block_q)


def head_operands(pooled_q: torch.Tensor, pooled_k: torch.Tensor, head_shared: bool):
    """The pooled operands that are scored against each other.

    selector.py, ``score_blocks``:
    * head_shared: the mean over heads of the pooled queries, and separately
      the mean over heads of the pooled keys (fp32), giving one selection head.
    * otherwise, with fewer kv heads than query heads (GQA), pooled kv head g
      serves query heads g*G .. g*G+G-1, G = Hq/Hkv (repeat_interleave order).

    Returns (qh, kh), each (B, H', N, D) fp32, where H' is 1 or Hq.
    """
    hq, hkv = pooled_q.shape[1], pooled_k.shape[1]
    if head_shared:
        qh = pooled_q.sum(dim=1, keepdim=True, dtype=torch.float32) / float(hq)
        kh = pooled_k.sum(dim=1, keepdim=True, dtype=torch.float32) / float(hkv)
        return qh, kh
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    group = hq // hkv
    kh = pooled_k[:, [h // group for h in range(hq)]]
    return pooled_q, kh


def score_blocks(q: torch.Tensor, k: torch.Tensor, block_q: int, block_kv: int,
                 head_shared: bool) -> np.ndarray:
    """fp32 tile scores s[b, h', i, j] = sum_d qh[b,h',i,d] * kh[b,h',j,d].

    selector.py, ``score_blocks``: no softmax scale and no softmax, since the
    per-row ranking does not change under either. The page splits the product
    into head chunks only to bound memory; that has no effect on the values and
    is not modelled here.
    """
    qh, kh = head_operands(pool_blocks(q, block_q), pool_blocks(k, block_kv), head_shared)
    a = qh.numpy().astype(np.float32, copy=False)
    b = kh.numpy().astype(np.float32, copy=False)
    return np.matmul(a, np.swapaxes(b, -1, -2)).astype(np.float32, copy=False)


def _as_mask(m, shape4) -> np.ndarray | None:
    """Optional mask as a 4-D bool array broadcastable to shape4 (dims 1 or full)."""
    if m is None:
        return None
    a = np.asarray(m)
    if a.ndim != 4:
        raise ValueError("masks are 4-D (B|1, H'|1, NQ, NK)")
    for got, want in zip(a.shape, shape4):
        if got not in (1, want):
            raise ValueError(f"mask shape {a.shape} does not broadcast to {shape4}")
    return a != 0


def keep_per_row(candidates_per_row: np.ndarray, budget: float) -> np.ndarray:
    """k_r = ceil(fl32(c_r) * fl32(budget)), as int64.

    selector.py, ``selection_plan``: the per-row count of candidates is an
    integer tensor multiplied by a Python float, which torch evaluates in
    float32; the product is rounded to float32 before the ceiling.
    """
    prod = np.asarray(candidates_per_row).astype(np.float32) * np.float32(budget)
    return np.ceil(prod.astype(np.float32)).astype(np.int64)


def selection_plan(nq: int, nk: int, block_q: int, block_kv: int, budget: float,
                   batch: int, heads: int, pins=None, drops=None, q_offset: int = 0):
    """What must be kept, what may be chosen and how many, from geometry and masks only.

    selector.py, ``selection_plan``:
      must       = diagonal OR pins
      forbidden  = drops (empty when absent)
      candidates = NOT must AND NOT forbidden
      c_r        = number of candidates in the row
      k_r        = ceil(c_r * budget) in fp32 (see ``keep_per_row``)
      dense      = every row has k_r >= c_r (the budget covers all candidates)

    Returns a dict of numpy arrays broadcast to (B, H', NQ, NK) / (B, H', NQ).
    """
    shape4 = (batch, heads, nq, nk)
    must = np.broadcast_to(diagonal_blocks(nq, nk, block_q, block_kv, q_offset), shape4)
    p = _as_mask(pins, shape4)
    if p is not None:
        must = must | p
    d = _as_mask(drops, shape4)
    forbidden = np.zeros(shape4, bool) if d is None else np.broadcast_to(d, shape4)
    must = np.broadcast_to(must, shape4)
    candidates = ~must & ~forbidden
    c = candidates.sum(axis=-1)
    k = keep_per_row(c, budget)
    dense = bool(np.all(k >= c))
    return dict(must=must, forbidden=forbidden, candidates=candidates, c=c, k=k, dense=dense)


def select_blocks(q: torch.Tensor, k: torch.Tensor, budget: float = 0.30, block_q: int = 128,
                  block_kv: int = 64, head_shared: bool = False, force: bool = False,
                  pins=None, drops=None, q_offset: int = 0):
    """Per query tile: the diagonal, the pins and the top-``k_r`` candidates, minus drops.

    selector.py, ``select_blocks``. q: (B, Hq, Sq, D), k: (B, Hkv, Skv, D), CPU
    tensors (fp32 or bf16). Returns None when the plan says the result would be
    dense and ``force`` is off (the caller then attends densely). Otherwise a dict:

      keep    int8 (B, H', NQ, NK)   1 = attend to the tile
      row_ptr int64 (B*H'*NQ + 1,)   CSR over rows r = (b*H' + h')*NQ + i
      col_idx int64 (nnz,)           kept kv tiles of each row, ascending
      scores  fp32 (B, H', NQ, NK)   pooled scores (before masking)
      c, k    int64 (B, H', NQ)      candidates and per-row budget
      near_tie bool (B, H', NQ)      the k-th and (k+1)-th candidate scores are
                                     within NEAR_TIE_REL of each other
    """
    bsz, hq, seq_q, _ = q.shape
    seq_kv = k.shape[-2]
    nq, nk = block_count(seq_q, block_q), block_count(seq_kv, block_kv)
    heads = 1 if head_shared else hq
    plan = selection_plan(nq, nk, block_q, block_kv, budget, bsz, heads, pins, drops, q_offset)
    if plan["dense"] and not force:
        return None

    scores = score_blocks(q, k, block_q, block_kv, head_shared)
    if not np.all(np.isfinite(scores)):
        raise ValueError("non-finite tile score: inputs must be finite")
    cand = plan["candidates"]
    kr = plan["k"]
    picked, near = rank_select(scores, cand, kr)
    keep = (plan["must"] | picked) & ~plan["forbidden"]

    keep8 = keep.astype(np.int8)
    row_ptr, col_idx = keep_to_csr(keep8)
    return dict(keep=keep8, row_ptr=row_ptr, col_idx=col_idx, scores=scores, c=plan["c"],
                k=kr, near_tie=near, must=np.ascontiguousarray(plan["must"]),
                forbidden=np.ascontiguousarray(plan["forbidden"]),
                block_q=block_q, block_kv=block_kv, seq_q=seq_q, seq_kv=seq_kv, heads=heads)


def rank_select(scores: np.ndarray, candidates: np.ndarray, k: np.ndarray):
    """Per row, pick the first k_r candidates in (score descending, kv index ascending) order.

    selector.py, ``select_blocks``: non-candidates are ranked behind every
    candidate (their score is replaced by -inf), the order is a stable
    descending sort (equal scores keep the lower kv index first, and -0.0
    equals +0.0), and a candidate is picked when its place in that order is
    below the row's budget k_r.

    Also returns the near-tie flag of each row with 0 < k_r < c_r: the k-th and
    (k+1)-th candidate scores differ by at most NEAR_TIE_REL relative to the
    larger magnitude of the two.

    scores: (..., NK) float; candidates: (..., NK) bool; k: (...) int.
    Returns (picked bool (..., NK), near_tie bool (...)).
    """
    nk = scores.shape[-1]
    ranked = np.where(candidates, scores, -np.inf).astype(np.float64)
    order = np.argsort(-ranked, axis=-1, kind="stable")
    first_k = np.arange(nk) < np.asarray(k)[..., None]
    picked_sorted = first_k & np.take_along_axis(candidates, order, axis=-1)
    picked = np.zeros(candidates.shape, bool)
    np.put_along_axis(picked, order, picked_sorted, axis=-1)

    sorted_scores = np.take_along_axis(ranked, order, axis=-1)
    c = candidates.sum(axis=-1)
    near = np.zeros(np.shape(k), bool)
    open_rows = (k > 0) & (k < c)
    if np.any(open_rows):
        idx = np.nonzero(open_rows)
        kk = np.asarray(k)[idx]
        s_k = sorted_scores[idx + (kk - 1,)]
        s_k1 = sorted_scores[idx + (kk,)]
        near[idx] = np.abs(s_k - s_k1) <= NEAR_TIE_REL * np.maximum(np.abs(s_k), np.abs(s_k1))
    return picked, near


def keep_to_csr(keep: np.ndarray):
    """Row-compressed list of kept kv tiles, ascending within each row.

    Rows are numbered r = (b*H' + h')*NQ + i (row-major over the keep array).
    The column order follows the ordered column indices the "Optimal ordering
    with block mask" thread describes for block masks.
    """
    flat = np.asarray(keep).reshape(-1, keep.shape[-1]) != 0
    counts = flat.sum(axis=1)
    row_ptr = np.zeros(flat.shape[0] + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(flat)[1].astype(np.int64)  # row-major: ascending per row
    return row_ptr, col_idx
