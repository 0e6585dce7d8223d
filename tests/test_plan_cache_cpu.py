"""The plan cache of nsa_select / nsa_select_sizes (host only, no GPU).

The selection page caches selection_plan under a key of its caller's choosing
plus tile counts, block sizes, budget and device, leaving the pin and drop
masks out of the key. The library keys on the whole request, masks included:
these tests check that a request differing only in one mask byte gets a plan
of its own, whose sizes and row offsets match the oracle's plan for its masks."""
import ctypes
import threading

import numpy as np
import pytest

import oracle
import top_kv_tile_amd as tkt
from top_kv_tile_amd import nsa as N


@pytest.fixture(autouse=True)
def fresh_cache():
    tkt.lib()
    tkt.nsa_plan_cache_config(8)
    tkt.nsa_plan_cache_clear()
    yield
    tkt.nsa_plan_cache_config(8)
    tkt.nsa_plan_cache_clear()


def _t(B, H, S, D=128):
    return N._Tensor(1, N.NSA_BF16, B, H, S, D)


def _sizes(q, k, spec, pins=None, drops=None):
    hold = []
    out = N._Sizes()
    nq, nk = -(-q.S // spec.block_q), -(-k.S // spec.block_kv)
    rows = q.B * (1 if spec.head_shared else q.H) * nq
    row_ptr = np.zeros(rows + 1, np.int32)
    st = tkt.lib().nsa_select_sizes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(spec._c()),
                                    N._mask(pins, hold), N._mask(drops, hold), ctypes.byref(out),
                                    row_ptr.ctypes.data)
    assert st == 0, tkt.nsa_status_string(st)
    return out, row_ptr


def _oracle_row_ptr(B, H, nq, nk, spec, pins, drops):
    plan = oracle.selection_plan(nq, nk, spec.block_q, spec.block_kv, spec.budget, B, H, pins, drops)
    counts = (plan["must"] & ~plan["forbidden"]).sum(-1) + np.minimum(plan["k"], plan["c"])
    return np.concatenate([[0], np.cumsum(counts.reshape(-1))]).astype(np.int64)


B, HQ, HKV, S, BQ, BKV = 2, 4, 2, 2048, 128, 64
NQ, NK = S // BQ, S // BKV
SPEC = tkt.SparseSpec(budget=0.25, block_q=BQ, block_kv=BKV)


def _masks(seed):
    rng = np.random.default_rng(seed)
    pins = (rng.random((1, 1, NQ, NK)) < 0.03).astype(np.int8)
    drops = (rng.random((B, HQ, NQ, NK)) < 0.05).astype(np.int8)
    return pins, drops


def test_repeat_hits_and_matches():
    pins, drops = _masks(0)
    a, ra = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    b, rb = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    assert tkt.nsa_plan_cache_stats() == (1, 1, 1)
    assert a.nnz == b.nnz and np.array_equal(ra, rb)
    assert np.array_equal(ra, _oracle_row_ptr(B, HQ, NQ, NK, SPEC, pins, drops))


def _candidate_flip(pins, drops):
    """(b, h, i, j) of a candidate tile (not must, not dropped) in a row where
    dropping it changes k_r, so a stale plan would have the wrong nnz."""
    plan = oracle.selection_plan(NQ, NK, BQ, BKV, SPEC.budget, B, HQ, pins, drops)
    for b in range(B):
        for h in range(HQ):
            for i in range(NQ):
                c = int(plan["c"][b, h, i])
                if c < 2 or int(oracle.keep_per_row(np.array([c - 1]), SPEC.budget)[0]) == int(plan["k"][b, h, i]):
                    continue
                js = np.nonzero(plan["candidates"][b, h, i])[0]
                return b, h, i, int(js[0])
    raise AssertionError("no row where one more drop changes k_r")


def test_one_drop_byte_gets_its_own_plan():
    pins, drops = _masks(1)
    a, ra = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    b_, h, i, j = _candidate_flip(pins, drops)
    drops2 = drops.copy()
    drops2[b_, h, i, j] = 1
    b, rb = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops2)
    assert tkt.nsa_plan_cache_stats() == (0, 2, 2)
    assert b.nnz != a.nnz
    assert np.array_equal(rb, _oracle_row_ptr(B, HQ, NQ, NK, SPEC, pins, drops2))
    # both stay cached and each request still finds its own plan
    a2, ra2 = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    assert a2.nnz == a.nnz and np.array_equal(ra2, ra)
    assert tkt.nsa_plan_cache_stats() == (1, 2, 2)


def test_one_pin_byte_gets_its_own_plan():
    pins, drops = _masks(2)
    a, _ = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    pins2 = pins.copy()
    plan = oracle.selection_plan(NQ, NK, BQ, BKV, SPEC.budget, B, HQ, pins, drops)
    free = np.argwhere(~plan["must"][0, 0] & (drops.max(axis=(0, 1)) == 0))
    pins2[0, 0, free[0][0], free[0][1]] = 1
    b, rb = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins2, drops)
    assert tkt.nsa_plan_cache_stats()[:2] == (0, 2)
    assert np.array_equal(rb, _oracle_row_ptr(B, HQ, NQ, NK, SPEC, pins2, drops))


def test_spec_shape_and_absent_masks_are_part_of_the_key():
    pins, drops = _masks(3)
    base, _ = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    other = tkt.SparseSpec(budget=0.3, block_q=BQ, block_kv=BKV)
    b, rb = _sizes(_t(B, HQ, S), _t(B, HKV, S), other, pins, drops)
    assert np.array_equal(rb, _oracle_row_ptr(B, HQ, NQ, NK, other, pins, drops))
    _sizes(_t(B, HQ, S - 64), _t(B, HKV, S - 64), SPEC)
    # no masks vs all-zero masks: same plan contents, different keys
    n1, r1 = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, None, None)
    n2, r2 = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, np.zeros((1, 1, NQ, NK), np.int8), None)
    assert np.array_equal(r1, r2)
    hits, misses, entries = tkt.nsa_plan_cache_stats()
    assert (hits, misses, entries) == (0, 5, 5)


def test_lru_eviction_and_capacity():
    tkt.nsa_plan_cache_config(2)
    reqs = [_masks(10 + x) for x in range(3)]
    for pins, drops in reqs:
        _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, pins, drops)
    assert tkt.nsa_plan_cache_stats() == (0, 3, 2)
    _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, *reqs[2])   # most recent: hit
    _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, *reqs[0])   # evicted first: miss
    assert tkt.nsa_plan_cache_stats() == (1, 4, 2)
    _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, *reqs[2])   # still held (used before reqs[0] came back)
    assert tkt.nsa_plan_cache_stats() == (2, 4, 2)
    tkt.nsa_plan_cache_config(1)
    assert tkt.nsa_plan_cache_stats()[2] == 1
    _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, *reqs[2])   # the most recently used entry was kept
    assert tkt.nsa_plan_cache_stats()[:2] == (3, 4)
    tkt.nsa_plan_cache_config(0)
    for _ in range(2):
        o, r = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, *reqs[1])
        assert np.array_equal(r, _oracle_row_ptr(B, HQ, NQ, NK, SPEC, *reqs[1]))
    assert tkt.nsa_plan_cache_stats() == (3, 6, 0)
    with pytest.raises(N.NsaError):
        tkt.nsa_plan_cache_config(-1)


def test_concurrent_callers():
    reqs = [_masks(20 + x) for x in range(3)]
    want = [_oracle_row_ptr(B, HQ, NQ, NK, SPEC, p, d) for p, d in reqs]
    errors = []

    def worker(t):
        try:
            for n in range(40):
                x = (t + n) % 3
                _, r = _sizes(_t(B, HQ, S), _t(B, HKV, S), SPEC, *reqs[x])
                if not np.array_equal(r, want[x]):
                    errors.append((t, n))
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors
    hits, misses, entries = tkt.nsa_plan_cache_stats()
    assert hits + misses == 8 * 40 and entries == 3 and misses >= 3


def test_large_masks_are_not_cached():
    """Each entry copies its masks: past 64 MiB of mask bytes a request is built
    per call (still correct) and not kept."""
    B2, Hq2, Hkv2, S2, bq2, bkv2 = 1, 72, 8, 65536, 128, 32
    nq2, nk2 = S2 // bq2, S2 // bkv2
    spec = tkt.SparseSpec(budget=0.1, block_q=bq2, block_kv=bkv2)
    drops = np.zeros((1, Hq2, nq2, nk2), np.int8)  # 72 MiB
    drops[:, :, :, 7] = 1
    for _ in range(2):
        out, r = _sizes(_t(B2, Hq2, S2), _t(B2, Hkv2, S2), spec, None, drops)
    assert tkt.nsa_plan_cache_stats() == (0, 2, 0)
    assert np.array_equal(r, _oracle_row_ptr(B2, Hq2, nq2, nk2, spec, None, drops))
