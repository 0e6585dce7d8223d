"""Seeded synthetic workloads shared by the tests, the bench and the oracle runs.

This module holds no arithmetic of the method (no pooling, scoring, ranking or
attention): it only draws inputs. Every tensor is drawn on the CPU with
``torch.Generator('cpu').manual_seed(seed)`` in fp32, in the order
q -> k structure -> k noise -> v -> drops, and then cast (round to nearest even)
to the workload dtype. Layout is (B, H, S, D), contiguous. Large tensors are
drawn one head at a time to bound host memory.

The named workloads reproduce the shapes the pages discuss: a tiny fp32 causal
case, plain MHA, causal GQA, an image-grid token set in Morton (Z-order) layout
(the ordering idea of "Optimal ordering with block mask", attention-gym issue
56) with head-shared scoring, and a long-context causal GQA case with a pinned
sink tile and random drops.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "morton_grid_coords",
           "tile_ranges_intersect"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    block_q: int
    block_kv: int
    budget: float
    head_shared: bool
    causal: bool
    dtype: str            # "f32" or "bf16"
    kind: str = "iid"     # "iid" | "morton_sinusoid" | "clusters"
    sink_pin: bool = False
    drop_frac: float = 0.0
    seed: int = 0
    grid: tuple = ()      # (rows, cols) for the Morton workload
    clusters: int = 0

    @property
    def nq(self) -> int:
        return -(-self.S // self.block_q)

    @property
    def nk(self) -> int:
        return -(-self.S // self.block_kv)

    @property
    def sel_heads(self) -> int:
        return 1 if self.head_shared else self.Hq

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny_causal_f32", B=1, Hq=2, Hkv=2, S=512, D=64, block_q=64, block_kv=32,
             budget=0.30, head_shared=False, causal=True, dtype="f32", seed=1000),
    Workload("mha_bf16_s8k", B=1, Hq=16, Hkv=16, S=8192, D=128, block_q=128, block_kv=64,
             budget=0.30, head_shared=False, causal=False, dtype="bf16", seed=1001),
    Workload("gqa_causal_bf16_s16k", B=2, Hq=32, Hkv=8, S=16384, D=128, block_q=128,
             block_kv=64, budget=0.25, head_shared=False, causal=True, dtype="bf16", seed=1002),
    Workload("grid2d_morton_shared_bf16", B=1, Hq=24, Hkv=24, S=32768, D=128, block_q=128,
             block_kv=64, budget=0.10, head_shared=True, causal=False, dtype="bf16",
             kind="morton_sinusoid", grid=(128, 256), seed=1003),
    Workload("long_causal_gqa_bf16_s128k", B=1, Hq=64, Hkv=8, S=131072, D=128, block_q=128,
             block_kv=64, budget=0.05, head_shared=False, causal=True, dtype="bf16",
             kind="clusters", clusters=64, sink_pin=True, drop_frac=0.01, seed=1004),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def morton_grid_coords(rows: int, cols: int):
    """(y, x) grid position of each Morton index m, for a rows x cols grid.

    Bits of x and y are interleaved (x in the even bits, y in the odd bits)
    while both have bits left; the remaining high bits of the longer side
    follow. For 128 x 256 this puts an 8 x 8 patch in each run of 64 indices.
    """
    ybits = int(math.log2(rows))
    xbits = int(math.log2(cols))
    if (1 << ybits) != rows or (1 << xbits) != cols:
        raise ValueError("grid sides must be powers of two")
    m = np.arange(rows * cols, dtype=np.int64)
    y = np.zeros_like(m)
    x = np.zeros_like(m)
    common = min(xbits, ybits)
    for i in range(common):
        x |= ((m >> (2 * i)) & 1) << i
        y |= ((m >> (2 * i + 1)) & 1) << i
    rest = m >> (2 * common)
    if xbits > ybits:
        x |= rest << common
    else:
        y |= rest << common
    return y, x


def tile_ranges_intersect(nq: int, nk: int, block_q: int, block_kv: int) -> np.ndarray:
    """(nq, nk) bool: the token ranges of query tile i and kv tile j intersect.

    Workload structure only: the drop recipe below never drops such a tile.
    """
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return (i * block_q < (j + 1) * block_kv) & (j * block_kv < (i + 1) * block_q)


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    pins: np.ndarray | None
    drops: np.ndarray | None
    meta: dict = field(default_factory=dict)


def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    """Draw q, k, v (CPU tensors in the workload dtype) and pins/drops (int8 or None)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    B, Hq, Hkv, S, D = w.B, w.Hq, w.Hkv, w.S, w.D
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    q = torch.empty((B, Hq, S, D), dtype=tdt)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = _cast(torch.randn((S, D), generator=g), w.dtype)

    k = torch.empty((B, Hkv, S, D), dtype=tdt)
    if w.kind == "iid":
        for b in range(B):
            for h in range(Hkv):
                k[b, h] = _cast(torch.randn((S, D), generator=g), w.dtype)
    elif w.kind == "morton_sinusoid":
        rows, cols = w.grid
        if rows * cols != S:
            raise ValueError("grid does not match S")
        yy, xx = morton_grid_coords(rows, cols)
        yy = torch.from_numpy(yy).to(torch.float64)
        xx = torch.from_numpy(xx).to(torch.float64)
        # k structure: per (b, head, d) an integer frequency pair (fy, fx) in
        # {0..3}^2 without (0, 0), and a phase in [0, 2 pi).
        pairs = torch.tensor([(a, c) for a in range(4) for c in range(4) if (a, c) != (0, 0)])
        pick = torch.randint(0, len(pairs), (B, Hkv, D), generator=g)
        phase = torch.rand((B, Hkv, D), generator=g, dtype=torch.float64) * (2 * math.pi)
        for b in range(B):
            for h in range(Hkv):
                f = pairs[pick[b, h]].to(torch.float64)          # (D, 2)
                arg = 2 * math.pi * (f[None, :, 0] * yy[:, None] / rows
                                     + f[None, :, 1] * xx[:, None] / cols) + phase[b, h][None, :]
                k[b, h] = _cast(torch.sin(arg).to(torch.float32), "f32").to(tdt)
        for b in range(B):
            for h in range(Hkv):
                noise = 0.3 * torch.randn((S, D), generator=g)
                k[b, h] = _cast(k[b, h].to(torch.float32) + noise, w.dtype)
    elif w.kind == "clusters":
        # k structure: per kv head, `clusters` centres ~ N(0, I_D) and one centre
        # per kv tile (drawn uniformly); each token of the tile is its centre plus
        # N(0, 1) noise, so pooling a tile keeps its centre.
        nk = w.nk
        centres = torch.randn((B, Hkv, w.clusters, D), generator=g)
        assign = torch.randint(0, w.clusters, (B, Hkv, nk), generator=g)
        for b in range(B):
            for h in range(Hkv):
                tok = assign[b, h].repeat_interleave(w.block_kv)[:S]
                base = centres[b, h][tok]
                noise = torch.randn((S, D), generator=g)
                k[b, h] = _cast(base + noise, w.dtype)
    else:
        raise ValueError(w.kind)

    v = torch.empty((B, Hkv, S, D), dtype=tdt)
    for b in range(B):
        for h in range(Hkv):
            v[b, h] = _cast(torch.randn((S, D), generator=g), w.dtype)

    nq, nk = w.nq, w.nk
    pins = None
    if w.sink_pin:
        pins = np.zeros((1, 1, nq, nk), np.int8)
        pins[..., 0] = 1
    drops = None
    if w.drop_frac > 0:
        eligible = ~tile_ranges_intersect(nq, nk, w.block_q, w.block_kv)
        if pins is not None:
            eligible &= pins[0, 0] == 0
        flat = np.flatnonzero(eligible)
        n_drop = int(round(w.drop_frac * flat.size))
        perm = torch.randperm(flat.size, generator=g)[:n_drop].numpy()
        drops = np.zeros((1, 1, nq, nk), np.int8)
        drops.reshape(-1)[flat[perm]] = 1
    return Inputs(q=q, k=k, v=v, pins=pins, drops=drops,
                  meta=dict(workload=w.name, seed=w.seed if seed is None else seed))
