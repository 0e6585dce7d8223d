"""Python binding of the C ABI in include/nsa.h (ctypes; argument marshalling only).

Every step of the path runs in the HIP library ``libnsa.so`` built next to this
file; torch supplies device memory and the current stream. There is no CPU or
eager fallback: when the library is missing every call raises.

Names follow the C ABI: ``nsa_select``, ``nsa_block_sparse_attn``,
``nsa_select_sizes``, ``nsa_pool_blocks``, ``nsa_score_blocks``,
``nsa_status_string``. ``SparseSpec`` and ``Selection`` mirror the SparseSpec and
BlockSelection of the page "automatic/modules/attention/sparse/selector.py".
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "SparseSpec", "Selection", "Sizes", "NsaError", "lib", "nsa_select_sizes", "nsa_select",
    "nsa_block_sparse_attn", "nsa_block_sparse_attn_bwd", "nsa_attn_bwd_workspace_size",
    "nsa_pool_blocks", "nsa_score_blocks", "nsa_status_string", "Plan", "nsa_plan_create",
    "nsa_select_planned", "nsa_schedule", "nsa_radial_blocks", "nsa_selection_density", "nsa_curve_order",
    "nsa_permute_tokens", "NSA_CURVE_MORTON", "NSA_CURVE_HILBERT", "nsa_decode_pool_update", "nsa_decode_select",
    "nsa_decode_attn", "nsa_decode_attn_static", "nsa_decode_attn_workspace_size", "nsa_plan_cache_config", "nsa_plan_cache_clear",
    "nsa_plan_cache_stats", "nsa_stage_timing_begin", "nsa_stage_timing_end", "LIB_PATH", "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnsa.so")
EXPORTS = ("nsa_select_sizes", "nsa_select", "nsa_block_sparse_attn", "nsa_attn_bwd_workspace_size",
           "nsa_block_sparse_attn_bwd", "nsa_pool_blocks", "nsa_score_blocks", "nsa_status_string",
           "nsa_last_hip_error", "nsa_version", "nsa_plan_create", "nsa_plan_sizes", "nsa_select_planned",
           "nsa_plan_destroy", "nsa_schedule", "nsa_radial_sizes", "nsa_radial_blocks", "nsa_selection_density",
           "nsa_curve_order", "nsa_permute_tokens", "nsa_decode_pool_update", "nsa_decode_select_sizes",
           "nsa_decode_select", "nsa_decode_attn", "nsa_decode_attn_workspace_size", "nsa_plan_cache_config",
           "nsa_plan_cache_clear", "nsa_plan_cache_stats", "nsa_decode_attn_static", "nsa_stage_timing_begin",
           "nsa_stage_timing_end", "nsa_plan_device_bytes", "nsa_plan_upload")

NSA_OK, NSA_DENSE = 0, 1
NSA_F32, NSA_BF16 = 0, 1
NSA_CURVE_MORTON, NSA_CURVE_HILBERT = 0, 1


class NsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {nsa_status_string(status)} (status {status})")


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("B", ctypes.c_int32),
                ("H", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32)]


class _Spec(ctypes.Structure):
    _fields_ = [("budget", ctypes.c_float), ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
                ("head_shared", ctypes.c_int32), ("force", ctypes.c_int32),
                ("score_chunk_bytes", ctypes.c_int64)]


class _Mask(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("b_dim", ctypes.c_int32), ("h_dim", ctypes.c_int32),
                ("nq", ctypes.c_int32), ("nk", ctypes.c_int32)]


class _Selection(ctypes.Structure):
    _fields_ = [("keep", ctypes.c_void_p), ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("col_capacity", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("NQ", ctypes.c_int32), ("NK", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
                ("seq_q", ctypes.c_int32), ("seq_kv", ctypes.c_int32), ("budget", ctypes.c_float)]


class _Sizes(ctypes.Structure):
    _fields_ = [("NQ", ctypes.c_int32), ("NK", ctypes.c_int32), ("sel_heads", ctypes.c_int32),
                ("dense", ctypes.c_int32), ("rows", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libnsa.so (raises if it was not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m top_kv_tile_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.nsa_select_sizes.argtypes = [P(_Tensor), P(_Tensor), P(_Spec), P(_Mask), P(_Mask), P(_Sizes),
                                       ctypes.c_void_p]
        L.nsa_select.argtypes = [P(_Tensor), P(_Tensor), P(_Spec), P(_Mask), P(_Mask), P(_Selection),
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.nsa_block_sparse_attn.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Selection), ctypes.c_int,
                                            P(_Tensor), ctypes.c_void_p, ctypes.c_void_p]
        L.nsa_attn_bwd_workspace_size.argtypes = [P(_Tensor), P(_Tensor), P(_Selection), P(ctypes.c_int64)]
        L.nsa_block_sparse_attn_bwd.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), ctypes.c_void_p,
                                                P(_Tensor), P(_Selection), ctypes.c_int, P(_Tensor), P(_Tensor),
                                                P(_Tensor), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.nsa_pool_blocks.argtypes = [P(_Tensor), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.nsa_score_blocks.argtypes = [P(_Tensor), P(_Tensor), P(_Spec), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
        L.nsa_plan_create.argtypes = [P(_Tensor), P(_Tensor), P(_Spec), P(_Mask), P(_Mask),
                                      P(ctypes.c_void_p)]
        L.nsa_plan_sizes.argtypes = [ctypes.c_void_p, P(_Sizes), ctypes.c_void_p]
        L.nsa_select_planned.argtypes = [ctypes.c_void_p, ctypes.c_void_p, P(_Tensor), P(_Tensor), P(_Selection),
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.nsa_plan_device_bytes.argtypes = [ctypes.c_void_p, P(ctypes.c_int64)]
        L.nsa_plan_upload.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.nsa_plan_destroy.argtypes = [ctypes.c_void_p]
        L.nsa_plan_destroy.restype = None
        L.nsa_plan_cache_config.argtypes = [ctypes.c_int32]
        L.nsa_plan_cache_clear.argtypes = []
        L.nsa_plan_cache_clear.restype = None
        L.nsa_plan_cache_stats.argtypes = [P(ctypes.c_int64), P(ctypes.c_int64), P(ctypes.c_int32)]
        L.nsa_schedule.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_int32,
                                   P(ctypes.c_double)]
        L.nsa_radial_sizes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P(_Spec), P(_Sizes),
                                       ctypes.c_void_p]
        L.nsa_radial_blocks.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P(_Spec), P(_Selection),
                                        ctypes.c_void_p]
        L.nsa_selection_density.argtypes = [P(_Selection), P(ctypes.c_double)]
        L.nsa_curve_order.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.nsa_permute_tokens.argtypes = [P(_Tensor), ctypes.c_void_p, ctypes.c_int32, P(_Tensor), ctypes.c_void_p]
        L.nsa_decode_pool_update.argtypes = [P(_Tensor), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        L.nsa_decode_select_sizes.argtypes = [P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_int32, P(_Spec),
                                              P(_Mask), P(_Mask), P(_Sizes), ctypes.c_void_p]
        L.nsa_decode_select.argtypes = [P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_int32, P(_Spec), P(_Mask),
                                        P(_Mask), P(_Selection), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.nsa_decode_attn.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_int32,
                                      P(_Selection), P(_Tensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]
        L.nsa_decode_attn_workspace_size.argtypes = [P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_int32,
                                                     P(_Selection), P(ctypes.c_int64)]
        L.nsa_decode_attn_static.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_int32,
                                             P(_Selection), P(_Tensor), ctypes.c_void_p, ctypes.c_void_p]
        L.nsa_stage_timing_begin.argtypes = []
        L.nsa_stage_timing_end.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(ctypes.c_int32)]
        L.nsa_status_string.argtypes = [ctypes.c_int]
        L.nsa_status_string.restype = ctypes.c_char_p
        L.nsa_version.restype = ctypes.c_char_p
        for name in ("nsa_select_sizes", "nsa_select", "nsa_block_sparse_attn", "nsa_attn_bwd_workspace_size",
                     "nsa_block_sparse_attn_bwd", "nsa_pool_blocks", "nsa_score_blocks", "nsa_last_hip_error",
                     "nsa_plan_create", "nsa_plan_sizes", "nsa_select_planned", "nsa_schedule", "nsa_radial_sizes",
                     "nsa_radial_blocks", "nsa_selection_density", "nsa_curve_order", "nsa_permute_tokens",
                     "nsa_decode_pool_update", "nsa_decode_select_sizes", "nsa_decode_select", "nsa_decode_attn",
                     "nsa_decode_attn_workspace_size", "nsa_plan_cache_config", "nsa_plan_cache_stats",
                     "nsa_decode_attn_static", "nsa_stage_timing_begin", "nsa_stage_timing_end",
                     "nsa_plan_device_bytes", "nsa_plan_upload"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def nsa_status_string(status: int) -> str:
    return lib().nsa_status_string(int(status)).decode()


@dataclass(frozen=True)
class SparseSpec:
    """Selection spec (defaults of SparseSpec on the selection page)."""
    budget: float = 0.30
    block_q: int = 128
    block_kv: int = 64
    head_shared: bool = False
    force: bool = False
    score_chunk_bytes: int = 256 << 20

    def _c(self) -> _Spec:
        return _Spec(float(self.budget), int(self.block_q), int(self.block_kv), int(bool(self.head_shared)),
                     int(bool(self.force)), int(self.score_chunk_bytes))


@dataclass
class Sizes:
    NQ: int
    NK: int
    sel_heads: int
    dense: bool
    rows: int
    nnz: int
    workspace_bytes: int


@dataclass
class Selection:
    """Keep flags and CSR of a block selection (device tensors)."""
    keep: torch.Tensor       # int8 (B, H', NQ, NK)
    row_ptr: torch.Tensor    # int32 (B*H'*NQ + 1)
    col_idx: torch.Tensor    # int32 (nnz)
    block_q: int
    block_kv: int
    budget: float
    seq_q: int
    seq_kv: int

    @property
    def shape(self):
        return tuple(self.keep.shape)

    @property
    def nnz(self) -> int:
        return int(self.col_idx.numel())

    def density(self) -> float:
        """Fraction of tiles kept (BlockSelection.density), from the known nnz: no device readback."""
        return nsa_selection_density(self)

    def _c(self) -> _Selection:
        B, H, NQ, NK = self.keep.shape
        return _Selection(self.keep.data_ptr(), self.row_ptr.data_ptr(),
                          self.col_idx.data_ptr() if self.col_idx.numel() else None,
                          self.col_idx.numel(), self.col_idx.numel(), B, H, NQ, NK, self.block_q,
                          self.block_kv, self.seq_q, self.seq_kv, float(self.budget))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NSA_F32
    if t.dtype == torch.bfloat16:
        return NSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _tensor(t: torch.Tensor) -> _Tensor:
    if t.dim() != 4:
        raise ValueError("tensors are 4-D (B, H, S, D)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    B, H, S, D = t.shape
    return _Tensor(t.data_ptr() if t.numel() else None, _dtype_code(t), B, H, S, D)


def _mask(m, keepalive: list):
    if m is None:
        return None
    a = np.ascontiguousarray(np.asarray(m).astype(np.int8, copy=False))
    if a.ndim != 4:
        raise ValueError("masks are 4-D (B|1, H'|1, NQ, NK)")
    keepalive.append(a)
    return ctypes.pointer(_Mask(a.ctypes.data if a.size else None, *a.shape))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, what: str):
    if status < 0:
        raise NsaError(status, what)
    return status


def nsa_select_sizes(q: torch.Tensor, k: torch.Tensor, spec: SparseSpec, pins=None, drops=None) -> Sizes:
    keep = []
    out = _Sizes()
    _check(lib().nsa_select_sizes(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(spec._c()),
                                  _mask(pins, keep), _mask(drops, keep), ctypes.byref(out), None),
           "nsa_select_sizes")
    return Sizes(out.NQ, out.NK, out.sel_heads, bool(out.dense), out.rows, out.nnz, out.workspace_bytes)


def nsa_select(q: torch.Tensor, k: torch.Tensor, spec: SparseSpec = SparseSpec(), pins=None, drops=None,
               stream=None, workspace: torch.Tensor | None = None):
    """select_blocks: returns a Selection, or None when the dense short circuit applies."""
    sizes = nsa_select_sizes(q, k, spec, pins, drops)
    if sizes.dense:
        return None
    dev = q.device
    B = q.shape[0]
    keep = torch.empty((B, sizes.sel_heads, sizes.NQ, sizes.NK), dtype=torch.int8, device=dev)
    row_ptr = torch.empty(sizes.rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(sizes.nnz, dtype=torch.int32, device=dev)
    if workspace is None or workspace.numel() < sizes.workspace_bytes:
        workspace = torch.empty(max(sizes.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    sel = Selection(keep, row_ptr, col_idx, spec.block_q, spec.block_kv, spec.budget, q.shape[2], k.shape[2])
    csel = sel._c()
    hold = []
    st = _check(lib().nsa_select(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(spec._c()),
                                 _mask(pins, hold), _mask(drops, hold), ctypes.byref(csel),
                                 ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)),
                "nsa_select")
    if st == NSA_DENSE:
        return None
    return sel


def nsa_block_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, selection: Selection | None,
                          causal: bool, stream=None, out: torch.Tensor | None = None,
                          lse: torch.Tensor | None = None):
    """Attention over the kept tiles; returns (out in q's dtype, lse fp32 (B, Hq, S))."""
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    csel = ctypes.byref(selection._c()) if selection is not None else None
    _check(lib().nsa_block_sparse_attn(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)),
                                       ctypes.byref(_tensor(v)), csel, int(bool(causal)),
                                       ctypes.byref(_tensor(out)), ctypes.c_void_p(lse.data_ptr()),
                                       _stream(stream)),
           "nsa_block_sparse_attn")
    return out, lse


def nsa_attn_bwd_workspace_size(q: torch.Tensor, k: torch.Tensor, selection: Selection | None) -> int:
    """Device workspace bytes nsa_block_sparse_attn_bwd needs."""
    n = ctypes.c_int64(0)
    csel = ctypes.byref(selection._c()) if selection is not None else None
    _check(lib().nsa_attn_bwd_workspace_size(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), csel,
                                             ctypes.byref(n)), "nsa_attn_bwd_workspace_size")
    return int(n.value)


def nsa_block_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                              lse: torch.Tensor, dout: torch.Tensor, selection: Selection | None, causal: bool,
                              stream=None, workspace: torch.Tensor | None = None, dq=None, dk=None, dv=None):
    """Gradients of nsa_block_sparse_attn; returns (dq, dk, dv) in q's dtype."""
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be contiguous fp32 (B, Hq, S)")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = nsa_attn_bwd_workspace_size(q, k, selection)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    csel = ctypes.byref(selection._c()) if selection is not None else None
    _check(lib().nsa_block_sparse_attn_bwd(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)),
                                           ctypes.byref(_tensor(v)), ctypes.byref(_tensor(out)),
                                           ctypes.c_void_p(lse.data_ptr()), ctypes.byref(_tensor(dout)), csel,
                                           int(bool(causal)), ctypes.byref(_tensor(dq)), ctypes.byref(_tensor(dk)),
                                           ctypes.byref(_tensor(dv)), ctypes.c_void_p(workspace.data_ptr()),
                                           workspace.numel() * workspace.element_size(), _stream(stream)),
           "nsa_block_sparse_attn_bwd")
    return dq, dk, dv


def nsa_pool_blocks(x: torch.Tensor, block: int, stream=None) -> torch.Tensor:
    n = -(-x.shape[2] // block)
    out = torch.empty((x.shape[0], x.shape[1], n, x.shape[3]), dtype=torch.float32, device=x.device)
    _check(lib().nsa_pool_blocks(ctypes.byref(_tensor(x)), int(block), ctypes.c_void_p(out.data_ptr()),
                                 _stream(stream)), "nsa_pool_blocks")
    return out


def nsa_score_blocks(q: torch.Tensor, k: torch.Tensor, spec: SparseSpec, stream=None) -> torch.Tensor:
    sizes = nsa_select_sizes(q, k, SparseSpec(budget=0.0, block_q=spec.block_q, block_kv=spec.block_kv,
                                              head_shared=spec.head_shared, force=True,
                                              score_chunk_bytes=spec.score_chunk_bytes))
    ws = torch.empty(max(sizes.workspace_bytes, 1), dtype=torch.uint8, device=q.device)
    s = torch.empty((q.shape[0], sizes.sel_heads, sizes.NQ, sizes.NK), dtype=torch.float32, device=q.device)
    _check(lib().nsa_score_blocks(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(spec._c()),
                                  ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  _stream(stream)), "nsa_score_blocks")
    return s


class Plan:
    """Host-side selection plan (nsa_plan_create): geometry, spec and mask contents, reusable across calls."""

    def __init__(self, handle: int, spec: SparseSpec, q_shape, k_shape, dtype):
        self._h = ctypes.c_void_p(handle)
        self.spec = spec
        self.q_shape, self.k_shape, self.dtype = tuple(q_shape), tuple(k_shape), dtype

    def sizes(self) -> Sizes:
        out = _Sizes()
        _check(lib().nsa_plan_sizes(self._h, ctypes.byref(out), None), "nsa_plan_sizes")
        return Sizes(out.NQ, out.NK, out.sel_heads, bool(out.dense), out.rows, out.nnz, out.workspace_bytes)

    def device_bytes(self) -> int:
        n = ctypes.c_int64(0)
        _check(lib().nsa_plan_device_bytes(self._h, ctypes.byref(n)), "nsa_plan_device_bytes")
        return n.value

    def upload(self, device, stream=None) -> torch.Tensor:
        """The plan's device image in a new uint8 tensor on `device` (nsa_plan_upload)."""
        img = torch.empty(max(self.device_bytes(), 1), dtype=torch.uint8, device=device)
        _check(lib().nsa_plan_upload(self._h, ctypes.c_void_p(img.data_ptr()), img.numel(), _stream(stream)),
               "nsa_plan_upload")
        return img

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h is not None and h.value and _LIB is not None:
            _LIB.nsa_plan_destroy(h)


def nsa_plan_create(q: torch.Tensor, k: torch.Tensor, spec: SparseSpec = SparseSpec(), pins=None,
                    drops=None) -> Plan:
    """Builds the selection plan for tensors shaped like q and k (read for shape and dtype only)."""
    h = ctypes.c_void_p()
    hold = []
    _check(lib().nsa_plan_create(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(spec._c()),
                                 _mask(pins, hold), _mask(drops, hold), ctypes.byref(h)), "nsa_plan_create")
    return Plan(h.value, spec, q.shape, k.shape, q.dtype)


def nsa_select_planned(plan: Plan, q: torch.Tensor, k: torch.Tensor, stream=None,
                       workspace: torch.Tensor | None = None, plan_dev: torch.Tensor | None = None):
    """nsa_select with a prebuilt plan; returns a Selection, or None when the plan is dense.

    plan_dev: the plan's device image from Plan.upload (None: uploaded by this call)."""
    sizes = plan.sizes()
    if sizes.dense:
        return None
    dev = q.device
    keep = torch.empty((q.shape[0], sizes.sel_heads, sizes.NQ, sizes.NK), dtype=torch.int8, device=dev)
    row_ptr = torch.empty(sizes.rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(sizes.nnz, dtype=torch.int32, device=dev)
    if workspace is None or workspace.numel() < sizes.workspace_bytes:
        workspace = torch.empty(max(sizes.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    spec = plan.spec
    sel = Selection(keep, row_ptr, col_idx, spec.block_q, spec.block_kv, spec.budget, q.shape[2], k.shape[2])
    csel = sel._c()
    img = ctypes.c_void_p(plan_dev.data_ptr()) if plan_dev is not None else None
    st = _check(lib().nsa_select_planned(plan._h, img, ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)),
                                         ctypes.byref(csel), ctypes.c_void_p(workspace.data_ptr()),
                                         workspace.numel(), _stream(stream)), "nsa_select_planned")
    return None if st == NSA_DENSE else sel


def nsa_plan_cache_config(capacity: int) -> None:
    """Plans kept by the cache of nsa_select / nsa_select_sizes (0 disables it)."""
    _check(lib().nsa_plan_cache_config(int(capacity)), "nsa_plan_cache_config")


def nsa_plan_cache_clear() -> None:
    """Drops every cached plan and zeroes the counters."""
    lib().nsa_plan_cache_clear()


def nsa_plan_cache_stats() -> tuple:
    """(hits, misses, entries) of the plan cache."""
    h, m, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(lib().nsa_plan_cache_stats(ctypes.byref(h), ctypes.byref(m), ctypes.byref(e)), "nsa_plan_cache_stats")
    return h.value, m.value, e.value


def nsa_schedule(steps: int, budget: float, bump: float = 0.0, bump_steps: int = 0) -> tuple:
    """Per-step budgets (schedule of the selection page)."""
    n = max(int(steps), 0)
    buf = (ctypes.c_double * max(n, 1))()
    _check(lib().nsa_schedule(int(steps), float(budget), float(bump), int(bump_steps), buf), "nsa_schedule")
    return tuple(buf[i] for i in range(n))


def nsa_radial_blocks(seq_q: int, seq_kv: int, density: float, spec: SparseSpec = SparseSpec(),
                      device="cuda:0", stream=None) -> Selection:
    """radial_blocks: the static band control at `density`; keep is (1, 1, NQ, NK)."""
    out = _Sizes()
    _check(lib().nsa_radial_sizes(int(seq_q), int(seq_kv), float(density), ctypes.byref(spec._c()),
                                  ctypes.byref(out), None), "nsa_radial_sizes")
    keep = torch.empty((1, 1, out.NQ, out.NK), dtype=torch.int8, device=device)
    row_ptr = torch.empty(out.NQ + 1, dtype=torch.int32, device=device)
    col_idx = torch.empty(out.nnz, dtype=torch.int32, device=device)
    sel = Selection(keep, row_ptr, col_idx, spec.block_q, spec.block_kv, float(density), int(seq_q), int(seq_kv))
    csel = sel._c()
    _check(lib().nsa_radial_blocks(int(seq_q), int(seq_kv), float(density), ctypes.byref(spec._c()),
                                   ctypes.byref(csel), _stream(stream)), "nsa_radial_blocks")
    return sel


def nsa_selection_density(sel: Selection) -> float:
    """BlockSelection.density from the selection's nnz (host only)."""
    d = ctypes.c_double()
    _check(lib().nsa_selection_density(ctypes.byref(sel._c()), ctypes.byref(d)), "nsa_selection_density")
    return d.value


def nsa_curve_order(kind, dims) -> np.ndarray:
    """perm[m] = raster index of the m-th grid point along the curve (NSA_CURVE_MORTON / NSA_CURVE_HILBERT)."""
    d = np.ascontiguousarray(np.asarray(dims, dtype=np.int32))
    n = int(np.prod(d.astype(np.int64))) if d.size else 0
    perm = np.empty(max(n, 1), np.int32)
    _check(lib().nsa_curve_order(int(kind), int(d.size), d.ctypes.data, perm.ctypes.data), "nsa_curve_order")
    return perm[:n]


def nsa_permute_tokens(x: torch.Tensor, perm: torch.Tensor, inverse: bool = False, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """Token rows gathered along perm (inverse=False) or scattered back (inverse=True)."""
    if perm.dtype != torch.int32 or not perm.is_contiguous():
        raise ValueError("perm must be contiguous int32")
    y = torch.empty_like(x) if out is None else out
    _check(lib().nsa_permute_tokens(ctypes.byref(_tensor(x)), ctypes.c_void_p(perm.data_ptr() if perm.numel() else 0),
                                    int(bool(inverse)), ctypes.byref(_tensor(y)), _stream(stream)),
           "nsa_permute_tokens")
    return y


def _tensor_f32(t: torch.Tensor) -> _Tensor:
    if t.dtype != torch.float32 or t.dim() != 4 or not t.is_contiguous():
        raise ValueError("pooled keys are a contiguous fp32 (B, Hkv, tiles, D) tensor")
    B, H, S, D = t.shape
    return _Tensor(t.data_ptr() if t.numel() else None, NSA_F32, B, H, S, D)


def nsa_decode_pool_update(k_cache: torch.Tensor, len_old: int, len_new: int, block_kv: int, pooled: torch.Tensor,
                           stream=None) -> torch.Tensor:
    """Refreshes the pooled-key cache for the tokens appended between len_old and len_new."""
    _check(lib().nsa_decode_pool_update(ctypes.byref(_tensor(k_cache)), int(len_old), int(len_new), int(block_kv),
                                        ctypes.c_void_p(pooled.data_ptr()), int(pooled.shape[2]), _stream(stream)),
           "nsa_decode_pool_update")
    return pooled


def nsa_decode_select(q: torch.Tensor, pooled_k: torch.Tensor, length: int, q_pos0: int,
                      spec: SparseSpec = SparseSpec(), pins=None, drops=None, stream=None,
                      workspace: torch.Tensor | None = None):
    """Selection for the new query tokens against the cache; a Selection, or None when dense."""
    hold = []
    out = _Sizes()
    pk = _tensor_f32(pooled_k)
    _check(lib().nsa_decode_select_sizes(ctypes.byref(_tensor(q)), ctypes.byref(pk), int(length), int(q_pos0),
                                         ctypes.byref(spec._c()), _mask(pins, hold), _mask(drops, hold),
                                         ctypes.byref(out), None), "nsa_decode_select_sizes")
    if out.dense:
        return None
    dev = q.device
    keep = torch.empty((q.shape[0], out.sel_heads, out.NQ, out.NK), dtype=torch.int8, device=dev)
    row_ptr = torch.empty(out.rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(out.nnz, dtype=torch.int32, device=dev)
    if workspace is None or workspace.numel() < out.workspace_bytes:
        workspace = torch.empty(max(out.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    sel = Selection(keep, row_ptr, col_idx, spec.block_q, spec.block_kv, spec.budget, q.shape[2], int(length))
    csel = sel._c()
    st = _check(lib().nsa_decode_select(ctypes.byref(_tensor(q)), ctypes.byref(pk), int(length), int(q_pos0),
                                        ctypes.byref(spec._c()), _mask(pins, hold), _mask(drops, hold),
                                        ctypes.byref(csel), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                        _stream(stream)), "nsa_decode_select")
    return None if st == NSA_DENSE else sel


def nsa_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, length: int, q_pos0: int,
                    selection: Selection | None, stream=None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Attention of the new query tokens over the kept tiles of the cache; returns (out, lse)."""
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    csel = ctypes.byref(selection._c()) if selection is not None else None
    need = ctypes.c_int64(0)
    _check(lib().nsa_decode_attn_workspace_size(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k_cache)),
                                                int(length), int(q_pos0), csel, ctypes.byref(need)),
           "nsa_decode_attn_workspace_size")
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().nsa_decode_attn(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k_cache)),
                                 ctypes.byref(_tensor(v_cache)), int(length), int(q_pos0), csel,
                                 ctypes.byref(_tensor(out)), ctypes.c_void_p(lse.data_ptr()),
                                 ctypes.c_void_p(workspace.data_ptr()),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "nsa_decode_attn")
    return out, lse


def nsa_decode_attn_workspace_size(q: torch.Tensor, k_cache: torch.Tensor, length: int, q_pos0: int,
                                   selection: Selection | None) -> int:
    """Bytes of split-partial workspace nsa_decode_attn needs for this request."""
    csel = ctypes.byref(selection._c()) if selection is not None else None
    need = ctypes.c_int64(0)
    _check(lib().nsa_decode_attn_workspace_size(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k_cache)),
                                                int(length), int(q_pos0), csel, ctypes.byref(need)),
           "nsa_decode_attn_workspace_size")
    return need.value


def nsa_decode_attn_static(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, length: int,
                           q_pos0: int, selection: Selection | None, out: torch.Tensor, lse: torch.Tensor,
                           stream=None):
    """nsa_decode_attn with the library's static scratch instead of a workspace.

    Allocates nothing: the caller passes ``out`` and ``lse``; returns them."""
    csel = ctypes.byref(selection._c()) if selection is not None else None
    _check(lib().nsa_decode_attn_static(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k_cache)),
                                        ctypes.byref(_tensor(v_cache)), int(length), int(q_pos0), csel,
                                        ctypes.byref(_tensor(out)), ctypes.c_void_p(lse.data_ptr()),
                                        _stream(stream)),
           "nsa_decode_attn_static")
    return out, lse


class _StageTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", ctypes.c_float)]


def nsa_stage_timing_begin():
    """Start recording stage events for the selection calls of this thread."""
    _check(lib().nsa_stage_timing_begin(), "nsa_stage_timing_begin")


def nsa_stage_timing_end(capacity: int = 1 << 14):
    """Stop recording; returns [(stage name, device ms)] in launch order."""
    buf = (_StageTime * capacity)()
    n = ctypes.c_int32(0)
    _check(lib().nsa_stage_timing_end(ctypes.cast(buf, ctypes.c_void_p), capacity, ctypes.byref(n)),
           "nsa_stage_timing_end")
    if n.value > capacity:
        raise NsaError(f"nsa_stage_timing_end: {n.value} stages recorded, capacity {capacity}")
    return [(buf[x].name.decode(), float(buf[x].ms)) for x in range(n.value)]
