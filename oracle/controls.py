"""Oracle for the selection page's controls: per-step budgets, the radial band,
and the kept-tile density.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page: "automatic/modules/attention/sparse/selector.py" -- ``schedule`` (per-step
budgets), ``radial_blocks`` (the static density-matched control the selector
is compared against) and ``BlockSelection.density``.

Arithmetic follows the page's types. Budgets are Python floats (fp64). The
radial band works on tile-centre distances held in float32, compares them with
a float64 bandwidth rounded to float32, and compares the float32 mean of the
kept flags with the requested density as float64.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["schedule", "radial_blocks", "density"]


def schedule(steps: int, budget: float, bump: float = 0.0, bump_steps: int = 0) -> tuple:
    """Per-step budgets: `budget` everywhere, raised to min(1, budget + bump) on
    the first and last `edge` steps, edge = min(bump_steps, ceil(steps / 2)).
    Without a positive bump, positive bump_steps and positive steps: the plain
    budget for max(steps, 0) steps."""
    if bump <= 0 or bump_steps <= 0 or steps <= 0:
        return tuple(float(budget) for _ in range(max(steps, 0)))
    raised = min(1.0, budget + bump)
    edge = min(bump_steps, math.ceil(steps / 2))
    out = []
    for i in range(steps):
        near_start = i < edge
        near_end = i >= steps - edge
        out.append(raised if (near_start or near_end) else float(budget))
    return tuple(out)


def _tile_centre_distance(seq_q: int, seq_kv: int, block_q: int, block_kv: int) -> np.ndarray:
    nq = -(-seq_q // block_q)
    nk = -(-seq_kv // block_kv)
    qc = (np.arange(nq, dtype=np.float32)[:, None] + np.float32(0.5)) * np.float32(block_q)
    kc = (np.arange(nk, dtype=np.float32)[None, :] + np.float32(0.5)) * np.float32(block_kv)
    return np.abs(qc - kc).astype(np.float32)


def _fraction_within(distance: np.ndarray, width: float) -> float:
    """float32 mean of (distance <= width), width rounded to float32, returned as a float."""
    inside = (distance <= np.float32(width)).astype(np.float32)
    with np.errstate(invalid="ignore"):  # no tiles: NaN, as the mean of an empty tensor
        return float(np.float32(inside.sum(dtype=np.float64)) / np.float32(inside.size))


def radial_blocks(seq_q: int, seq_kv: int, density: float, block_q: int, block_kv: int) -> np.ndarray:
    """Band of tiles around the diagonal at the requested density, (1, 1, NQ, NK) int8.

    A tile is kept when the distance between the centres of its query and kv
    token ranges is at most the bandwidth. The bandwidth is found by 40 halvings
    of [0, max(seq_q, seq_kv)]: a trial width whose kept fraction falls short of
    `density` raises the lower end, any other lowers the upper end, and the band
    uses the final upper end."""
    distance = _tile_centre_distance(seq_q, seq_kv, block_q, block_kv)
    low, high = 0.0, float(max(seq_q, seq_kv))
    for _ in range(40):
        mid = (low + high) / 2
        if _fraction_within(distance, mid) < density:
            low = mid
        else:
            high = mid
    keep = (distance <= np.float32(high)).astype(np.int8)
    return keep[None, None]


def density(keep) -> float:
    """Fraction of tiles kept (BlockSelection.density)."""
    keep = np.asarray(keep)
    return float((keep != 0).sum()) / max(keep.size, 1)
