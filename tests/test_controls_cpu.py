"""Host-only entry points of the controls and plan reuse, against the oracle (no GPU needed)."""
import ctypes

import numpy as np
import pytest

import oracle
import top_kv_tile_amd as tkt
from top_kv_tile_amd import nsa as N


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(N.LIB_PATH):
        from top_kv_tile_amd import build
        build.build()
    return tkt.lib()


@pytest.mark.parametrize("args", [(5, 0.3, 0.2, 1), (5, 0.3, 0.2, 3), (4, 0.9, 0.5, 1), (6, 0.1, 0.05, 2),
                                  (3, 0.25, 0.0, 2), (3, 0.25, 0.1, 0), (0, 0.25, 0.1, 2), (-2, 0.25, 0.1, 2),
                                  (1, 0.4, 0.1, 5), (11, 0.05, 0.3, 4), (12, 1.0, 0.2, 3)])
def test_schedule_matches_oracle(L, args):
    assert tkt.nsa_schedule(*args) == oracle.schedule(*args)


@pytest.mark.parametrize("seq_q,seq_kv,bq,bkv,dens", [
    (1024, 1024, 128, 64, 0.1), (1000, 1000, 128, 64, 0.05), (777, 777, 64, 32, 0.3), (900, 700, 64, 32, 0.2),
    (60000, 60000, 600, 7, 0.037), (131072, 131072, 128, 64, 0.05), (512, 512, 64, 64, 0.0),
    (300, 300, 128, 64, 1.0), (0, 0, 128, 64, 0.5),
])
def test_radial_sizes_match_oracle(L, seq_q, seq_kv, bq, bkv, dens):
    spec = tkt.SparseSpec(block_q=bq, block_kv=bkv)
    ref = oracle.radial_blocks(seq_q, seq_kv, dens, bq, bkv)[0, 0]
    nq, nk = ref.shape
    out = N._Sizes()
    row_ptr = np.zeros(nq + 1, np.int32)
    st = L.nsa_radial_sizes(seq_q, seq_kv, dens, ctypes.byref(spec._c()), ctypes.byref(out), row_ptr.ctypes.data)
    assert st == 0
    assert (out.NQ, out.NK, out.sel_heads, out.rows, out.dense) == (nq, nk, 1, nq, 0)
    assert out.nnz == int(ref.sum())
    assert np.array_equal(row_ptr, np.concatenate([[0], np.cumsum(ref.sum(1))]))


def test_radial_rejects_bad_spec(L):
    out = N._Sizes()
    assert L.nsa_radial_sizes(100, 100, 0.5, ctypes.byref(tkt.SparseSpec(block_q=0)._c()), ctypes.byref(out),
                              None) == -6
    assert L.nsa_radial_sizes(-1, 100, 0.5, ctypes.byref(tkt.SparseSpec()._c()), ctypes.byref(out), None) == -6
    assert L.nsa_radial_sizes(100, 100, 0.5, None, ctypes.byref(out), None) == -1


def _t(B, H, S, D, dtype=N.NSA_BF16):
    return N._Tensor(1, dtype, B, H, S, D)


@pytest.mark.parametrize("B,Hq,Hkv,S,bq,bkv,budget,shared,pshape,dshape", [
    (2, 4, 2, 1000, 128, 64, 0.25, False, (1, 1), (2, 4)),
    (1, 6, 3, 777, 128, 64, 0.10, True, (1, 1), (1, 1)),
    (1, 64, 8, 131072, 128, 64, 0.05, False, (1, 1), (1, 1)),
])
def test_plan_sizes_equal_select_sizes(L, B, Hq, Hkv, S, bq, bkv, budget, shared, pshape, dshape):
    nq, nk = -(-S // bq), -(-S // bkv)
    H = 1 if shared else Hq
    rng = np.random.default_rng(S)
    pins = (rng.random(pshape + (nq, nk)) < 0.02).astype(np.int8)
    drops = (rng.random(dshape + (nq, nk)) < 0.02).astype(np.int8)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv, head_shared=shared)
    hold = []
    q, k = _t(B, Hq, S, 128), _t(B, Hkv, S, 128)
    a = N._Sizes()
    rp_a = np.zeros(B * H * nq + 1, np.int32)
    assert L.nsa_select_sizes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(spec._c()), N._mask(pins, hold),
                              N._mask(drops, hold), ctypes.byref(a), rp_a.ctypes.data) == 0
    h = ctypes.c_void_p()
    assert L.nsa_plan_create(ctypes.byref(q), ctypes.byref(k), ctypes.byref(spec._c()), N._mask(pins, hold),
                             N._mask(drops, hold), ctypes.byref(h)) == 0
    pins[:] = 1  # the plan copied what it needs
    b = N._Sizes()
    rp_b = np.zeros(B * H * nq + 1, np.int32)
    assert L.nsa_plan_sizes(h, ctypes.byref(b), rp_b.ctypes.data) == 0
    for f in ("NQ", "NK", "sel_heads", "dense", "rows", "nnz", "workspace_bytes"):
        assert getattr(a, f) == getattr(b, f), f
    assert np.array_equal(rp_a, rp_b)
    # shape mismatch is rejected before anything is enqueued
    sel = N._Selection(keep=1, row_ptr=1, col_idx=1, col_capacity=1 << 40)
    assert L.nsa_select_planned(h, None, ctypes.byref(_t(B, Hq, S + 1, 128)), ctypes.byref(k), ctypes.byref(sel),
                                None, 0, None) == -2
    assert L.nsa_select_planned(h, None, ctypes.byref(_t(B, Hq, S, 128, N.NSA_F32)), ctypes.byref(k),
                                ctypes.byref(sel), None, 0, None) == -3
    # the device image: size from the plan (row offsets + bit-packed masks, 256-byte sections),
    # a missing, misaligned or short buffer is rejected before anything is enqueued
    n = ctypes.c_int64(-1)
    assert L.nsa_plan_device_bytes(h, ctypes.byref(n)) == 0
    sec = lambda x: -(-x // 256) * 256  # noqa: E731
    nkw = -(-nk // 64)
    want = (sec(4 * (B * H * nq + 1)) + sec(8 * int(np.prod(pshape)) * nq * nkw)
            + sec(8 * int(np.prod(dshape)) * nq * nkw))
    assert n.value == want
    assert L.nsa_plan_upload(h, None, n.value, None) == -5
    assert L.nsa_plan_upload(h, ctypes.c_void_p(4096 + 16), n.value, None) == -5
    assert L.nsa_plan_upload(h, ctypes.c_void_p(4096), n.value - 1, None) == -5
    assert L.nsa_plan_upload(None, ctypes.c_void_p(4096), n.value, None) == -1
    assert L.nsa_plan_device_bytes(h, None) == -1
    assert L.nsa_select_planned(h, ctypes.c_void_p(4096 + 8), ctypes.byref(_t(B, Hq, S, 128)), ctypes.byref(k),
                                ctypes.byref(sel), None, 0, None) == -5
    L.nsa_plan_destroy(h)
    L.nsa_plan_destroy(None)


def test_plan_create_validates(L):
    h = ctypes.c_void_p()
    assert L.nsa_plan_create(ctypes.byref(_t(1, 4, 256, 128)), ctypes.byref(_t(1, 3, 256, 128)),
                             ctypes.byref(tkt.SparseSpec()._c()), None, None, ctypes.byref(h)) == -2
    assert not h.value


def test_selection_density_from_nnz(L):
    sel = N._Selection(keep=1, row_ptr=1, col_idx=1, nnz=30, B=2, H=3, NQ=4, NK=5)
    d = ctypes.c_double()
    assert L.nsa_selection_density(ctypes.byref(sel), ctypes.byref(d)) == 0
    assert d.value == 30 / 120
    empty = N._Selection(nnz=0, B=1, H=1, NQ=0, NK=0)
    assert L.nsa_selection_density(ctypes.byref(empty), ctypes.byref(d)) == 0 and d.value == 0.0


@pytest.mark.parametrize("dims", [(4, 4), (2, 2, 2), (128, 256), (5, 7), (3, 4, 5), (16, 16, 16), (1, 9), (64,),
                                  (6, 10, 12)])
def test_curve_orders_match_oracle(L, dims):
    assert np.array_equal(tkt.nsa_curve_order(tkt.NSA_CURVE_MORTON, dims), oracle.morton_order(dims))
    assert np.array_equal(tkt.nsa_curve_order(tkt.NSA_CURVE_HILBERT, dims), oracle.hilbert_order(dims))


def test_curve_order_validation(L):
    d = np.array([4, 4], np.int32)
    out = np.zeros(16, np.int32)
    assert L.nsa_curve_order(2, 2, d.ctypes.data, out.ctypes.data) == -6
    assert L.nsa_curve_order(0, 0, d.ctypes.data, out.ctypes.data) == -4
    assert L.nsa_curve_order(0, 2, None, out.ctypes.data) == -1
    assert L.nsa_curve_order(0, 2, np.array([4, -1], np.int32).ctypes.data, out.ctypes.data) == -2
    assert L.nsa_curve_order(0, 2, np.array([0, 5], np.int32).ctypes.data, None) == 0  # empty grid


def test_permute_validation(L):
    x = N._Tensor(1, N.NSA_BF16, 1, 2, 16, 128)
    y = N._Tensor(2, N.NSA_BF16, 1, 2, 16, 128)
    assert L.nsa_permute_tokens(ctypes.byref(x), None, 0, ctypes.byref(y), None) == -1
    assert L.nsa_permute_tokens(ctypes.byref(x), 1, 0, ctypes.byref(N._Tensor(2, N.NSA_F32, 1, 2, 16, 128)),
                                None) == -3
    assert L.nsa_permute_tokens(ctypes.byref(x), 1, 0, ctypes.byref(N._Tensor(2, N.NSA_BF16, 1, 2, 15, 128)),
                                None) == -2
    assert L.nsa_permute_tokens(ctypes.byref(x), 1, 0, ctypes.byref(x), None) == -4          # in place
    odd = N._Tensor(16, N.NSA_BF16, 1, 2, 16, 48)
    assert L.nsa_permute_tokens(ctypes.byref(odd), 1, 0, ctypes.byref(N._Tensor(32, N.NSA_BF16, 1, 2, 16, 48)),
                                None) == -4


def _dec_sizes(L, q, pk, length, pos0, spec, pins=None, drops=None, row_ptr=None):
    hold = []
    out = N._Sizes()
    st = L.nsa_decode_select_sizes(ctypes.byref(q), ctypes.byref(pk), length, pos0, ctypes.byref(spec._c()),
                                   N._mask(pins, hold), N._mask(drops, hold), ctypes.byref(out),
                                   row_ptr.ctypes.data if row_ptr is not None else None)
    return st, out


@pytest.mark.parametrize("n,length,bq,bkv,budget", [(1, 1000, 128, 64, 0.3), (5, 4097, 128, 64, 0.05),
                                                    (64, 700, 32, 64, 0.25), (1, 1, 128, 64, 0.3)])
def test_decode_plan_matches_oracle(L, n, length, bq, bkv, budget):
    B, Hq, Hkv, D = 1, 4, 2, 128
    q = N._Tensor(1, N.NSA_BF16, B, Hq, n, D)
    pk = N._Tensor(1, N.NSA_F32, B, Hkv, 4096, D)
    pos0 = length - n
    nq, nk = -(-n // bq), -(-length // bkv)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv, force=True)
    row_ptr = np.zeros(B * Hq * nq + 1, np.int32)
    st, out = _dec_sizes(L, q, pk, length, pos0, spec, row_ptr=row_ptr)
    assert st == 0
    plan = oracle.selection_plan(nq, nk, bq, bkv, budget, B, Hq, q_offset=pos0)
    counts = (plan["must"] & ~plan["forbidden"]).sum(-1) + np.minimum(plan["k"], plan["c"])
    assert (out.NQ, out.NK) == (nq, nk)
    assert np.array_equal(row_ptr, np.concatenate([[0], np.cumsum(counts.reshape(-1))]))


def test_decode_validation(L):
    q = N._Tensor(1, N.NSA_BF16, 1, 4, 2, 128)
    pk = N._Tensor(1, N.NSA_F32, 1, 2, 16, 128)
    spec = tkt.SparseSpec()
    assert _dec_sizes(L, q, pk, 1000, 998, spec)[0] == 0
    assert _dec_sizes(L, q, pk, 1000, 999, spec)[0] == -2          # queries past the cache
    assert _dec_sizes(L, q, pk, 1025, 1000, spec)[0] == -2         # 17 tiles > 16 pooled
    assert _dec_sizes(L, q, N._Tensor(1, N.NSA_BF16, 1, 2, 16, 128), 1000, 998, spec)[0] == -3
    assert _dec_sizes(L, q, N._Tensor(1, N.NSA_F32, 1, 3, 16, 128), 1000, 998, spec)[0] == -2
    kc = N._Tensor(1, N.NSA_BF16, 1, 2, 512, 128)
    assert L.nsa_decode_pool_update(ctypes.byref(kc), 10, 5, 64, 1, 8, None) == -2
    assert L.nsa_decode_pool_update(ctypes.byref(kc), 0, 513, 64, 1, 9, None) == -2
    assert L.nsa_decode_pool_update(ctypes.byref(kc), 0, 512, 64, 1, 7, None) == -2
    assert L.nsa_decode_pool_update(ctypes.byref(kc), 0, 512, 0, 1, 8, None) == -6
    assert L.nsa_decode_pool_update(ctypes.byref(kc), 7, 7, 64, None, 8, None) == 0   # nothing appended
    out = N._Tensor(1, N.NSA_BF16, 1, 4, 2, 128)
    A = L.nsa_decode_attn
    big = 1 << 30
    assert A(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(kc), 600, 100, None, ctypes.byref(out), 1, 1, big,
             None) == -2
    assert A(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(kc), 500, 499, None, ctypes.byref(out), 1, 1, big,
             None) == -2
    assert A(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(kc), 500, 10, None, ctypes.byref(out), None, 1, big,
             None) == -1
    n = ctypes.c_int64(-1)
    assert L.nsa_decode_attn_workspace_size(ctypes.byref(q), ctypes.byref(kc), 500, 10, None, ctypes.byref(n)) == 0
    assert n.value == 0  # 8 tiles per row: too few to split
    kl = N._Tensor(1, N.NSA_BF16, 1, 2, 2048, 128)
    assert L.nsa_decode_attn_workspace_size(ctypes.byref(q), ctypes.byref(kl), 2000, 10, None, ctypes.byref(n)) == 0
    # 4 rows of 32 tiles: 4 splits of 8 tiles, fp32 partials of D values plus (reference, sum) per split
    assert n.value == 4 * 2 * 4 * 128 * 4 + 256
    assert A(ctypes.byref(q), ctypes.byref(kl), ctypes.byref(kl), 2000, 10, None, ctypes.byref(out), 1, 1,
             n.value - 1, None) == -5
