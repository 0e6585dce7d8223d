"""Pins for the control oracle (schedule, radial band, density).

The selection page prints no values for these functions, so the pins are:
* schedule: values worked out by hand from its definition (raise the first
  and last edge steps, cap at 1), and the invariants it states (at most two
  distinct values, symmetric, length = steps);
* radial band: a brute-force characterisation that does not bisect. Among
  the distinct tile-centre distances, take the smallest one whose kept
  fraction (float32 mean, as the page computes it) reaches the density. The
  band keeps exactly the tiles within it. Also: every row is one contiguous
  run, the band always contains the tile nearest the diagonal for density 1,
  and it is empty for density 0 when no centres coincide;
* density: a direct count.
"""
import numpy as np
import pytest

from oracle import controls


@pytest.mark.parametrize("args,want", [
    ((5, 0.3, 0.2, 1), (0.5, 0.3, 0.3, 0.3, 0.5)),
    ((5, 0.3, 0.2, 3), (0.5,) * 5),                     # edge = min(3, ceil(5/2)) covers all
    ((4, 0.9, 0.5, 1), (1.0, 0.9, 0.9, 1.0)),          # raised budget is capped at 1
    ((6, 0.1, 0.05, 2), (0.15000000000000002, 0.15000000000000002, 0.1, 0.1,
                         0.15000000000000002, 0.15000000000000002)),  # 0.1 + 0.05 in fp64
    ((3, 0.25, 0.0, 2), (0.25, 0.25, 0.25)),           # no bump
    ((3, 0.25, 0.1, 0), (0.25, 0.25, 0.25)),           # no bump steps
    ((0, 0.25, 0.1, 2), ()),
    ((-2, 0.25, 0.1, 2), ()),
    ((1, 0.4, 0.1, 5), (0.5,)),
])
def test_schedule_hand_values(args, want):
    got = controls.schedule(*args)
    assert got == want


@pytest.mark.parametrize("steps,bump_steps", [(1, 1), (7, 2), (8, 3), (10, 20), (9, 4)])
def test_schedule_invariants(steps, bump_steps):
    got = controls.schedule(steps, 0.3, 0.1, bump_steps)
    assert len(got) == steps
    assert len(set(got)) <= 2
    assert got == tuple(reversed(got))
    edge = min(bump_steps, -(-steps // 2))
    assert sum(1 for x in got if x != 0.3) == min(steps, 2 * edge)


def _brute_force_band(seq_q, seq_kv, dens, bq, bkv):
    nq, nk = -(-seq_q // bq), -(-seq_kv // bkv)
    qc = np.array([(i + 0.5) * bq for i in range(nq)])
    kc = np.array([(j + 0.5) * bkv for j in range(nk)])
    dist = np.abs(qc[:, None] - kc[None, :]).astype(np.float32)   # exact: half-integers below 2^24
    n = dist.size
    values, counts = np.unique(dist.reshape(-1), return_counts=True)
    within = np.cumsum(counts)                                    # tiles with distance <= values[t]
    frac = (within.astype(np.float32) / np.float32(n)).astype(np.float64)
    ok = np.nonzero(~(frac < dens))[0]
    if ok.size == 0:  # density above 1: the bisection ends at the largest width
        return np.ones((nq, nk), np.int8)
    return (dist <= values[ok[0]]).astype(np.int8)


@pytest.mark.parametrize("seq,bq,bkv,dens", [
    (1024, 128, 64, 0.10), (1024, 128, 64, 0.25), (1000, 128, 64, 0.05), (777, 64, 32, 0.3),
    (2048, 64, 64, 0.5), (512, 128, 128, 0.125), (4096, 128, 64, 0.01), (300, 128, 64, 0.99),
    (60000, 600, 7, 0.037),  # centre distances 0.5 apart over 60000 tokens: needs every halving
])
def test_radial_matches_brute_force(seq, bq, bkv, dens):
    keep = controls.radial_blocks(seq, seq, dens, bq, bkv)
    assert keep.shape[:2] == (1, 1) and keep.dtype == np.int8
    want = _brute_force_band(seq, seq, dens, bq, bkv)
    assert np.array_equal(keep[0, 0], want)
    assert controls.density(keep) >= dens - 1e-7


@pytest.mark.parametrize("seq_q,seq_kv,bq,bkv", [(1024, 1024, 128, 64), (900, 700, 64, 32)])
def test_radial_rows_are_contiguous_runs(seq_q, seq_kv, bq, bkv):
    for dens in (0.05, 0.2, 0.6):
        keep = controls.radial_blocks(seq_q, seq_kv, dens, bq, bkv)[0, 0]
        for row in keep:
            idx = np.nonzero(row)[0]
            if idx.size:
                assert idx[-1] - idx[0] + 1 == idx.size


def test_radial_extremes():
    # centres at 128 i + 64 and 64 j + 32 never coincide: density 0 keeps nothing
    assert controls.radial_blocks(1024, 1024, 0.0, 128, 64).sum() == 0
    assert np.all(controls.radial_blocks(1024, 1024, 1.0, 128, 64) == 1)
    # equal block sizes: centres coincide on the diagonal, density 0 keeps exactly it
    k0 = controls.radial_blocks(512, 512, 0.0, 64, 64)[0, 0]
    assert np.array_equal(k0, np.eye(8, dtype=np.int8))


def test_density_counts():
    keep = np.zeros((2, 3, 4, 5), np.int8)
    keep[0, 1, 2, 3] = 1
    keep[1, 2, :, 0] = 7
    assert controls.density(keep) == 5 / 120
    assert controls.density(np.zeros((1, 1, 0, 0), np.int8)) == 0.0
