"""CPU-side checks of the C ABI: the library loads, exports every declared symbol,
and its host-only plan and argument validation behave (no GPU needed: nothing
here reaches a launch)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from top_kv_tile_amd import nsa as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(N.LIB_PATH):
        from top_kv_tile_amd import build
        build.build()
    return tkt.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "nsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(nsa_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(N.EXPORTS) == set(names)


def test_status_strings(L):
    for s in (0, 1, -1, -2, -3, -4, -5, -6, -7, -8, 99):
        assert isinstance(tkt.nsa_status_string(s), str) and tkt.nsa_status_string(s)
    assert L.nsa_version() == b"0.1.0"


def _t(B, H, S, D, dtype=N.NSA_BF16, data=1):
    return N._Tensor(data, dtype, B, H, S, D)


def _sizes(q, k, spec, pins=None, drops=None, row_ptr=None):
    hold = []
    out = N._Sizes()
    st = tkt.lib().nsa_select_sizes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(spec._c()),
                                    N._mask(pins, hold), N._mask(drops, hold), ctypes.byref(out),
                                    row_ptr.ctypes.data if row_ptr is not None else None)
    return st, out


@pytest.mark.parametrize("B,Hq,Hkv,S,bq,bkv,budget,shared,pshape,dshape", [
    (1, 2, 2, 512, 64, 32, 0.30, False, None, None),
    (2, 4, 2, 1000, 128, 64, 0.25, False, (1, 1), (2, 4)),
    (1, 6, 3, 777, 128, 64, 0.10, True, (1, 1), (1, 1)),
    (2, 3, 1, 4096, 96, 48, 0.5, False, (2, 1), (1, 3)),
    (1, 64, 8, 131072, 128, 64, 0.05, False, (1, 1), (1, 1)),
])
def test_plan_sizes_and_row_ptr_match_oracle(L, B, Hq, Hkv, S, bq, bkv, budget, shared, pshape, dshape):
    nq, nk = -(-S // bq), -(-S // bkv)
    H = 1 if shared else Hq
    rng = np.random.default_rng(S)
    pins = None if pshape is None else (rng.random(pshape + (nq, nk)) < 0.02).astype(np.int8)
    drops = None if dshape is None else (rng.random(dshape + (nq, nk)) < 0.02).astype(np.int8)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv, head_shared=shared)
    row_ptr = np.zeros(B * H * nq + 1, np.int32)
    st, out = _sizes(_t(B, Hq, S, 128), _t(B, Hkv, S, 128), spec, pins, drops, row_ptr)
    assert st == 0
    plan = oracle.selection_plan(nq, nk, bq, bkv, budget, B, H, pins, drops)
    counts = (plan["must"] & ~plan["forbidden"]).sum(-1) + np.minimum(plan["k"], plan["c"])
    want = np.concatenate([[0], np.cumsum(counts.reshape(-1))])
    assert (out.NQ, out.NK, out.sel_heads, out.rows) == (nq, nk, H, B * H * nq)
    assert out.nnz == want[-1]
    assert np.array_equal(row_ptr, want)
    assert out.dense == int(plan["dense"])
    assert out.workspace_bytes > 0 and out.workspace_bytes % 256 == 0


def test_dense_decision_and_force(L):
    q, k = _t(1, 2, 512, 64), _t(1, 2, 512, 64)
    st, out = _sizes(q, k, tkt.SparseSpec(budget=1.0, block_q=64, block_kv=32))
    assert st == 0 and out.dense == 1
    st, out = _sizes(q, k, tkt.SparseSpec(budget=1.0, block_q=64, block_kv=32, force=True))
    assert st == 0 and out.dense == 0 and out.nnz == 2 * 8 * 16  # every tile of both heads
    st, out = _sizes(_t(1, 2, 0, 64), _t(1, 2, 0, 64, data=None), tkt.SparseSpec())
    assert st == 0 and out.dense == 1 and out.rows == 0
    # a finite budget far above 1 keeps every candidate, like budget 1
    # (k_r is clamped to c_r before its integer conversion)
    for budget in (1.5, 1e30, 3.0e38):
        st, out = _sizes(q, k, tkt.SparseSpec(budget=budget, block_q=64, block_kv=32, force=True))
        assert st == 0 and out.dense == 0 and out.nnz == 2 * 8 * 16, budget
        st, out = _sizes(q, k, tkt.SparseSpec(budget=budget, block_q=64, block_kv=32))
        assert st == 0 and out.dense == 1, budget


@pytest.mark.parametrize("mutate,code", [
    (lambda q, k, s: (q, N._Tensor(1, N.NSA_BF16, 1, 3, 256, 128), s), -2),   # Hq % Hkv
    (lambda q, k, s: (q, N._Tensor(1, N.NSA_F32, 1, 2, 256, 128), s), -3),    # dtype mismatch
    (lambda q, k, s: (q, N._Tensor(1, 7, 1, 2, 256, 128), s), -3),            # bad dtype code
    (lambda q, k, s: (q, N._Tensor(1, N.NSA_BF16, 2, 2, 256, 128), s), -2),   # batch mismatch
    (lambda q, k, s: (q, N._Tensor(1, N.NSA_BF16, 1, 2, 256, 64), s), -2),    # D mismatch
    (lambda q, k, s: (N._Tensor(1, N.NSA_BF16, 1, 4, 256, 96), N._Tensor(1, N.NSA_BF16, 1, 2, 256, 96), s), -4),
    (lambda q, k, s: (q, k, tkt.SparseSpec(budget=-0.1)), -6),
    (lambda q, k, s: (q, k, tkt.SparseSpec(budget=float("nan"))), -6),
    (lambda q, k, s: (q, k, tkt.SparseSpec(budget=float("inf"))), -6),
    (lambda q, k, s: (q, k, tkt.SparseSpec(budget=1e39)), -6),         # inf once rounded to fp32
    (lambda q, k, s: (q, k, tkt.SparseSpec(block_q=0)), -6),
    (lambda q, k, s: (q, k, tkt.SparseSpec(score_chunk_bytes=-1)), -6),
    (lambda q, k, s: (N._Tensor(None, N.NSA_BF16, 1, 4, 256, 128), k, s), -1),
    (lambda q, k, s: (N._Tensor(1, N.NSA_BF16, 1, 4, 64 * 8192, 128), N._Tensor(1, N.NSA_BF16, 1, 2, 64 * 8192, 128), s), -4),
])
def test_select_sizes_validation(L, mutate, code):
    q, k, s = mutate(_t(1, 4, 256, 128), _t(1, 2, 256, 128), tkt.SparseSpec())
    st, _ = _sizes(q, k, s)
    assert st == code


@pytest.mark.parametrize("pshape,code", [((1, 1, 2, 4), 0), ((2, 1, 2, 4), 0), ((3, 1, 2, 4), -2),
                                          ((1, 4, 2, 4), 0), ((1, 2, 2, 4), -2), ((1, 1, 3, 4), -2),
                                          ((1, 1, 2, 5), -2)])
def test_mask_broadcast_validation(L, pshape, code):
    pins = np.zeros(pshape, np.int8)
    st, _ = _sizes(_t(2, 4, 256, 128), _t(2, 2, 256, 128), tkt.SparseSpec(), pins=pins)
    assert st == code


def test_select_and_attn_reject_before_launch(L):
    """Invalid calls return an error code without touching the device."""
    hold = []
    sel = N._Selection()
    q = _t(1, 4, 256, 128)
    k = _t(1, 3, 256, 128)
    st = L.nsa_select(ctypes.byref(q), ctypes.byref(k), ctypes.byref(tkt.SparseSpec()._c()), None, None,
                      ctypes.byref(sel), None, 0, None)
    assert st == -2
    # capacity too small (valid shapes, so the plan runs, but nothing launches)
    k = _t(1, 2, 256, 128)
    sel = N._Selection(keep=1, row_ptr=1, col_idx=1, col_capacity=1)
    st = L.nsa_select(ctypes.byref(q), ctypes.byref(k), ctypes.byref(tkt.SparseSpec()._c()), None, None,
                      ctypes.byref(sel), None, 0, None)
    assert st == -8
    # workspace too small
    sel = N._Selection(keep=1, row_ptr=1, col_idx=1, col_capacity=1 << 20)
    st = L.nsa_select(ctypes.byref(q), ctypes.byref(k), ctypes.byref(tkt.SparseSpec()._c()), None, None,
                      ctypes.byref(sel), ctypes.c_void_p(256), 16, None)
    assert st == -5
    # dense short circuit: outputs untouched, nothing enqueued
    st = L.nsa_select(ctypes.byref(q), ctypes.byref(k), ctypes.byref(tkt.SparseSpec(budget=1.0)._c()), None,
                      None, ctypes.byref(sel), None, 0, None)
    assert st == 1
    # attention: dtype mismatch, shape mismatch, causal with Sq != Skv, unsupported D
    out = _t(1, 4, 256, 128)
    lse = ctypes.c_void_p(1)
    A = L.nsa_block_sparse_attn
    assert A(ctypes.byref(q), ctypes.byref(_t(1, 2, 256, 128, N.NSA_F32)), ctypes.byref(k), None, 1,
             ctypes.byref(out), lse, None) == -3
    assert A(ctypes.byref(q), ctypes.byref(_t(1, 2, 256, 128)), ctypes.byref(_t(1, 2, 255, 128)), None, 1,
             ctypes.byref(out), lse, None) == -2
    assert A(ctypes.byref(q), ctypes.byref(_t(1, 2, 300, 128)), ctypes.byref(_t(1, 2, 300, 128)), None, 1,
             ctypes.byref(out), lse, None) == -4
    q96 = _t(1, 4, 256, 96)
    assert A(ctypes.byref(q96), ctypes.byref(_t(1, 2, 256, 96)), ctypes.byref(_t(1, 2, 256, 96)), None, 0,
             ctypes.byref(_t(1, 4, 256, 96)), lse, None) == -4
    assert A(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), None, 0, ctypes.byref(out), None, None) == -1
    bad_sel = N._Selection(keep=1, row_ptr=1, col_idx=1, nnz=5, B=1, H=3, NQ=2, NK=4, block_q=128,
                           block_kv=64, seq_q=256, seq_kv=256)
    assert A(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(bad_sel), 0, ctypes.byref(out),
             lse, None) == -2


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(N, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(N, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        N.lib()


def _bwd(L, q, k, v, out, lse, do, sel, causal, dq, dk, dv, ws, nbytes):
    return L.nsa_block_sparse_attn_bwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(out), lse,
                                       ctypes.byref(do), ctypes.byref(sel) if sel is not None else None, causal,
                                       ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ws, nbytes, None)


def test_backward_workspace_size(L):
    q, k = _t(2, 4, 1000, 128), _t(2, 2, 1000, 128)
    n = ctypes.c_int64(-1)
    assert L.nsa_attn_bwd_workspace_size(ctypes.byref(q), ctypes.byref(k), None, ctypes.byref(n)) == 0
    a = lambda x: (x + 255) // 256 * 256
    assert n.value == a(2 * 4 * 1000 * 4)  # Delta only
    sel = N._Selection(keep=1, row_ptr=1, col_idx=1, nnz=300, B=2, H=4, NQ=8, NK=16, block_q=128, block_kv=64,
                       seq_q=1000, seq_kv=1000)
    assert L.nsa_attn_bwd_workspace_size(ctypes.byref(q), ctypes.byref(k), ctypes.byref(sel), ctypes.byref(n)) == 0
    # Delta, column counts per quarter of the query tiles, col_ptr, per-2048-column block sums + total, row_idx
    cols = 2 * 4 * 16
    assert n.value == (a(2 * 4 * 1000 * 4) + a(cols * 4 * 4) + a((cols + 1) * 4) + a((-(-cols // 2048) + 1) * 4)
                       + a(300 * 4))
    bad = N._Selection(keep=1, row_ptr=1, col_idx=1, nnz=300, B=2, H=3, NQ=8, NK=16, block_q=128, block_kv=64,
                       seq_q=1000, seq_kv=1000)
    assert L.nsa_attn_bwd_workspace_size(ctypes.byref(q), ctypes.byref(k), ctypes.byref(bad), ctypes.byref(n)) == -2
    assert L.nsa_attn_bwd_workspace_size(ctypes.byref(q), ctypes.byref(k), None, None) == -1


def test_backward_rejects_before_launch(L):
    q, k = _t(1, 4, 256, 128), _t(1, 2, 256, 128)
    lse = ctypes.c_void_p(1)
    ws = ctypes.c_void_p(256)
    big = 1 << 30
    ok = dict(q=q, k=k, v=_t(1, 2, 256, 128), out=_t(1, 4, 256, 128), lse=lse, do=_t(1, 4, 256, 128), sel=None,
              causal=1, dq=_t(1, 4, 256, 128), dk=_t(1, 2, 256, 128), dv=_t(1, 2, 256, 128), ws=ws, nbytes=big)

    def call(**over):
        args = dict(ok)
        args.update(over)
        return _bwd(L, **args)

    assert call(v=_t(1, 2, 256, 128, N.NSA_F32)) == -3             # dtype mismatch
    assert call(dq=_t(1, 4, 255, 128)) == -2                        # dq shape
    assert call(dk=_t(1, 4, 256, 128)) == -2                        # dk heads
    assert call(lse=None) == -1                                     # missing lse
    assert call(nbytes=16) == -5                                    # workspace too small
    assert call(ws=None) == -5
    assert call(q=_t(1, 4, 256, 96), out=_t(1, 4, 256, 96), do=_t(1, 4, 256, 96), dq=_t(1, 4, 256, 96),
                k=_t(1, 2, 256, 96), v=_t(1, 2, 256, 96), dk=_t(1, 2, 256, 96), dv=_t(1, 2, 256, 96)) == -4
    sel_nokeep = N._Selection(keep=None, row_ptr=1, col_idx=1, nnz=5, B=1, H=4, NQ=2, NK=4, block_q=128,
                              block_kv=64, seq_q=256, seq_kv=256)
    assert call(sel=sel_nokeep) == -1
    sel_badnnz = N._Selection(keep=1, row_ptr=1, col_idx=1, nnz=-3, B=1, H=4, NQ=2, NK=4, block_q=128,
                              block_kv=64, seq_q=256, seq_kv=256)
    assert call(sel=sel_badnnz) == -2


def test_decode_attn_static_rejects_before_launch(L):
    """The allocation-free decode call checks its request against the static
    buffer before any HIP call: a split-partial need above
    NSA_DECODE_SCRATCH_BYTES is NSA_ERR_WORKSPACE, bad shapes as nsa_decode_attn."""
    limit = 16 << 20
    hdr = open(os.path.join(ROOT, "include", "nsa.h")).read()
    assert re.search(r"#define NSA_DECODE_SCRATCH_BYTES \(16u << 20\)", hdr)
    S = L.nsa_decode_attn_static
    lse = ctypes.c_void_p(1)
    # 32 query heads x 32 new tokens over a 128k cache, dense: 64 splits of fp32 partials
    q = _t(1, 32, 32, 128)
    kc = _t(1, 32, 131072, 128)
    need = ctypes.c_int64(0)
    assert L.nsa_decode_attn_workspace_size(ctypes.byref(q), ctypes.byref(kc), 131072, 131072 - 32, None,
                                            ctypes.byref(need)) == 0
    assert need.value > limit
    assert S(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(kc), 131072, 131072 - 32, None,
             ctypes.byref(_t(1, 32, 32, 128)), lse, None) == -5
    # shape and argument errors come first, as in nsa_decode_attn
    assert S(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(kc), 131073, 0, None,
             ctypes.byref(_t(1, 32, 32, 128)), lse, None) == -2
    assert S(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(kc), 131072, 131072 - 32, None,
             ctypes.byref(_t(1, 32, 32, 128)), None, None) == -1
    assert S(ctypes.byref(q), ctypes.byref(_t(1, 32, 131072, 128, N.NSA_F32)), ctypes.byref(kc), 131072, 0,
             None, ctypes.byref(_t(1, 32, 32, 128)), lse, None) == -3


NULL_ARG = -1  # NSA_ERR_NULL_ARG (include/nsa.h)


def test_stage_timing_host_side(L):
    """Begin / end with nothing recorded needs no GPU: an empty list, and NULL_ARG
    for a missing count or a missing buffer with capacity > 0."""
    assert L.nsa_stage_timing_begin() == N.NSA_OK
    n = ctypes.c_int32(-1)
    assert L.nsa_stage_timing_end(None, 0, ctypes.byref(n)) == N.NSA_OK
    assert n.value == 0
    assert L.nsa_stage_timing_end(None, 0, None) == NULL_ARG
    assert L.nsa_stage_timing_end(None, 4, ctypes.byref(n)) == NULL_ARG
    tkt.nsa_stage_timing_begin()
    assert tkt.nsa_stage_timing_end() == []
