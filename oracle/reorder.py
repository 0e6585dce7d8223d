"""Oracle for token reordering along space-filling curves.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page: "Optimal ordering with block mask" (attention-gym issue 56). For tokens
laid out on a grid (pixels of an image, voxels of a video), the order of the
sequence decides how many (query tile, kv tile) blocks a local attention
pattern touches. The thread suggests a Morton (Z-order) curve, cheap to
compute, or a Hilbert curve, applied once before a series of attention calls.

An order is returned as `perm`: perm[m] is the raster index (last axis
fastest) of the token placed at position m. Reordering gathers
y[..., m, :] = x[..., perm[m], :]; undoing it scatters back.

* Morton: the key of a grid point interleaves the bits of its coordinates,
  bit b of axis a (a = 0 the fastest axis) going to bit b * n + a of the key
  (n axes); positions follow increasing keys.
* Hilbert: the key is the Hilbert index of the point in the enclosing
  2^p x ... x 2^p cube, computed with J. Skilling's transpose method
  ("Programming the Hilbert curve", AIP Conf. Proc. 707, 2004): Gray-decode
  the coordinate bits from the top level down, exchanging or inverting the
  low bits per level, then Gray-encode. The index is read from the transposed
  form bit level by bit level, the slowest axis contributing the high bit of
  each level. Grids that are not full cubes keep the order of the cube's
  curve restricted to their points.
"""
from __future__ import annotations

import numpy as np

__all__ = ["morton_order", "hilbert_order", "apply_order", "undo_order"]


def _coords(dims):
    """(S, n) coordinates of the raster positions, axis order as `dims`."""
    grids = np.meshgrid(*[np.arange(d) for d in dims], indexing="ij")
    return np.stack([g.reshape(-1) for g in grids], axis=1).astype(np.int64)


def _bits_needed(dims) -> int:
    m = max(dims) if len(dims) else 1
    p = 0
    while (1 << p) < m:
        p += 1
    return max(p, 1)


def morton_order(dims) -> np.ndarray:
    dims = tuple(int(d) for d in dims)
    n = len(dims)
    c = _coords(dims)
    p = _bits_needed(dims)
    key = np.zeros(c.shape[0], np.int64)
    for b in range(p):
        for a in range(n):
            axis = n - 1 - a  # a = 0 is the fastest (last) axis
            key |= ((c[:, axis] >> b) & 1) << (b * n + a)
    return np.argsort(key, kind="stable").astype(np.int64)


def _hilbert_key(point, p: int) -> int:
    """Hilbert index of one point (tuple of n coordinates in [0, 2^p))."""
    x = [int(v) for v in point]
    n = len(x)
    # coordinates to the transposed index
    m = 1 << (p - 1)
    q = m
    while q > 1:
        mask = q - 1
        for i in range(n):
            if x[i] & q:
                x[0] ^= mask               # invert the low bits of the first axis
            else:
                t = (x[0] ^ x[i]) & mask   # exchange the low bits with the first axis
                x[0] ^= t
                x[i] ^= t
        q >>= 1
    for i in range(1, n):                  # Gray encode
        x[i] ^= x[i - 1]
    t = 0
    q = m
    while q > 1:
        if x[n - 1] & q:
            t ^= q - 1
        q >>= 1
    for i in range(n):
        x[i] ^= t
    # read the index: bit level by bit level, axis 0 giving the high bit of each level
    key = 0
    for b in range(p - 1, -1, -1):
        for i in range(n):
            key = (key << 1) | ((x[i] >> b) & 1)
    return key


def hilbert_order(dims) -> np.ndarray:
    dims = tuple(int(d) for d in dims)
    c = _coords(dims)
    p = _bits_needed(dims)
    keys = np.array([_hilbert_key(tuple(pt), p) for pt in c], np.int64)
    return np.argsort(keys, kind="stable").astype(np.int64)


def apply_order(x: np.ndarray, perm) -> np.ndarray:
    """y[..., m, :] = x[..., perm[m], :]."""
    return np.asarray(x)[..., np.asarray(perm), :]


def undo_order(y: np.ndarray, perm) -> np.ndarray:
    """x with x[..., perm[m], :] = y[..., m, :]."""
    y = np.asarray(y)
    out = np.empty_like(y)
    out[..., np.asarray(perm), :] = y
    return out
