"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Small, seeded cases that span several tiles, ragged tails, GQA, head-shared
scoring, pins and drops (drops winning over the diagonal, empty rows), the
dense short circuit, sequences shorter than a block, the widest supported row
(NK = 4096), all-tied scores, and both attention kernels (bf16 MFMA and the
general fp32/bf16 kernel).
"""
import math

import zlib

import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from parity_util import check_attention, check_selection, run_case, say, to_dev

pytestmark = pytest.mark.gpu


def _qkv(B, Hq, Hkv, S, D, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, S, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, S, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, S, D, generator=g).to(dtype)
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S,D,block", [(300, 64, 64), (100, 128, 128), (1000, 128, 64), (64, 256, 32)])
def test_pool_blocks(dtype, S, D, block):
    say(f"pool dtype={dtype} S={S} D={D} block={block}")
    g = torch.Generator().manual_seed(S + D)
    x = torch.randn(2, 3, S, D, generator=g).to(dtype)
    got = tkt.nsa_pool_blocks(to_dev(x), block).cpu().double()
    ref = oracle.pool_blocks(x, block).double()
    n = block
    bound = 2 * n * 2.0 ** -24 * x.abs().max().item() + 1e-30
    assert got.shape == ref.shape
    assert (got - ref).abs().max().item() <= bound


@pytest.mark.parametrize("Hq,Hkv,shared,S,D,bq,bkv", [
    (4, 4, False, 2000, 128, 128, 64), (8, 2, False, 2000, 128, 128, 64), (6, 3, True, 2000, 128, 128, 64),
    # more than 64 query tiles (the split-operand bf16 kernel), ragged in both block dimensions
    (4, 2, False, 20000, 128, 128, 64), (2, 1, False, 9000, 64, 64, 32), (2, 2, True, 12000, 256, 128, 64),
    # 567 blocks of 128 x 256: more than the persistent grid holds, and not a multiple of 8
    (63, 7, False, 40000, 64, 128, 64),
])
def test_score_blocks(Hq, Hkv, shared, S, D, bq, bkv):
    say(f"scores Hq={Hq} Hkv={Hkv} shared={shared} S={S} D={D} bq={bq} bkv={bkv}")
    q, k, _ = _qkv(1, Hq, Hkv, S, D, seed=Hq * 7 + Hkv, dtype=torch.bfloat16)
    spec = tkt.SparseSpec(block_q=bq, block_kv=bkv, head_shared=shared)
    got = tkt.nsa_score_blocks(to_dev(q), to_dev(k), spec).cpu().numpy().astype(np.float64)
    ref = oracle.score_blocks(q, k, bq, bkv, shared).astype(np.float64)
    qh, kh = oracle.head_operands(oracle.pool_blocks(q, bq), oracle.pool_blocks(k, bkv), shared)
    mag = np.abs(qh.double().numpy()) @ np.swapaxes(np.abs(kh.double().numpy()), -1, -2)
    assert got.shape == ref.shape
    assert np.all(np.abs(got - ref) <= 4 * D * 2.0 ** -24 * mag + 1e-30)


@pytest.mark.parametrize("S,bkv", [(9000, 64), (16384, 64)])
def test_score_blocks_wide_range(S, bkv):
    """The many-row score kernel splits each pooled fp32 value into three bf16
    terms. Operands whose dimensions span 2^-20 .. 2^20 in magnitude (fp32
    inputs, so the pooled values carry all 24 significant bits) must still
    score within the fp32 bound: against the oracle, and against the exact
    (fp64) product of the library's own pooled operands, which isolates the
    score kernel's error. 141 kv tiles leave ragged 256-key blocks, 256 whole ones."""
    D, bq = 128, 128
    say(f"scores wide range S={S} bkv={bkv}")
    g = torch.Generator().manual_seed(S)
    scale = torch.exp2(torch.randint(-20, 21, (1, 1, 1, D), generator=g).float())
    q = torch.randn(1, 4, S, D, generator=g) * scale
    k = torch.randn(1, 2, S, D, generator=g) / scale.flip(-1)
    spec = tkt.SparseSpec(block_q=bq, block_kv=bkv)
    got = tkt.nsa_score_blocks(to_dev(q), to_dev(k), spec).cpu().numpy().astype(np.float64)
    ref = oracle.score_blocks(q, k, bq, bkv, False).astype(np.float64)
    qh, kh = oracle.head_operands(oracle.pool_blocks(q, bq), oracle.pool_blocks(k, bkv), False)
    mag = np.abs(qh.double().numpy()) @ np.swapaxes(np.abs(kh.double().numpy()), -1, -2)
    assert got.shape == ref.shape and got.shape[2] > 64
    assert np.all(np.abs(got - ref) <= 4 * D * 2.0 ** -24 * mag + 1e-30)
    pq = tkt.nsa_pool_blocks(to_dev(q), bq).cpu()
    pk = tkt.nsa_pool_blocks(to_dev(k), bkv).cpu()
    gq, gk = oracle.head_operands(pq, pk, False)
    qd, kd = gq.double().numpy(), np.swapaxes(gk.double().numpy(), -1, -2)
    exact, gmag = qd @ kd, np.abs(qd) @ np.abs(kd)
    assert np.all(np.abs(got - exact) <= 2 * D * 2.0 ** -24 * gmag + 1e-30)


CASES = [
    # name, B, Hq, Hkv, S, D, bq, bkv, budget, shared, causal, dtype
    ("tiny_f32_causal", 1, 2, 2, 512, 64, 64, 32, 0.30, False, True, torch.float32),
    ("bf16_gqa_causal_ragged", 2, 4, 2, 1000, 128, 128, 64, 0.30, False, True, torch.bfloat16),
    ("bf16_shared_noncausal_ragged", 1, 4, 4, 777, 128, 128, 64, 0.25, True, False, torch.bfloat16),
    ("bf16_d64_bq64_gqa8", 1, 8, 1, 2048, 64, 64, 64, 0.20, False, True, torch.bfloat16),
    ("bf16_bq32", 1, 2, 2, 640, 128, 32, 64, 0.40, False, True, torch.bfloat16),
    ("bf16_bq96_ragged", 1, 2, 1, 1000, 128, 96, 64, 0.30, False, True, torch.bfloat16),
    ("bf16_d64_bq96", 1, 4, 2, 1000, 64, 96, 64, 0.30, False, True, torch.bfloat16),
    ("bf16_general_kernel_bkv32", 1, 2, 1, 700, 64, 64, 32, 0.30, False, True, torch.bfloat16),
    ("f32_d128_noncausal", 1, 2, 2, 600, 128, 128, 64, 0.50, False, False, torch.float32),
    ("bf16_budget0", 1, 2, 2, 1024, 128, 128, 64, 0.0, False, False, torch.bfloat16),
    ("bf16_nk100", 1, 2, 2, 6400, 128, 128, 64, 0.10, False, False, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_select_and_attention(case):
    name, B, Hq, Hkv, S, D, bq, bkv, budget, shared, causal, dtype = case
    say(f"case {name}")
    q, k, v = _qkv(B, Hq, Hkv, S, D, seed=zlib.crc32(name.encode()) % 10000, dtype=dtype)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv, head_shared=shared)
    rep = run_case(q, k, v, spec, causal, where=name)
    say(f"  {rep}")


def test_pins_drops_broadcast_and_drop_wins():
    """Pins per batch, drops per head, a dropped diagonal tile (empty causal rows)."""
    B, Hq, Hkv, S, D, bq, bkv = 2, 4, 2, 1024, 128, 128, 64
    say("pins/drops broadcast")
    q, k, v = _qkv(B, Hq, Hkv, S, D, seed=77, dtype=torch.bfloat16)
    nq, nk = 8, 16
    rng = np.random.default_rng(5)
    pins = (rng.random((B, 1, nq, nk)) < 0.1).astype(np.int8)
    drops = (rng.random((1, Hq, nq, nk)) < 0.1).astype(np.int8)
    drops[0, 1, 3, 6] = 1  # diagonal tiles of row 3 are kv 6 and 7
    drops[0, 1, 3, 7] = 1
    pins[:, :, 3, :] = 0
    spec = tkt.SparseSpec(budget=0.3, block_q=bq, block_kv=bkv)
    rep = run_case(q, k, v, spec, True, pins=pins, drops=drops, where="pins_drops")
    say(f"  {rep}")


def test_force_budget_one_equals_dense():
    """budget 1 + force keeps everything; the GPU result equals the GPU dense call and the oracle."""
    say("force budget 1")
    q, k, v = _qkv(1, 4, 2, 1000, 128, seed=3, dtype=torch.bfloat16)
    spec = tkt.SparseSpec(budget=1.0, block_q=128, block_kv=64, force=True)
    rep = run_case(q, k, v, spec, True, where="force1")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sel = tkt.nsa_select(qd, kd, spec)
    assert int(sel.keep.min().item()) == 1
    o1, l1 = tkt.nsa_block_sparse_attn(qd, kd, vd, sel, True)
    o2, l2 = tkt.nsa_block_sparse_attn(qd, kd, vd, None, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    say(f"  {rep}")


def test_dense_short_circuit():
    say("dense short circuit")
    q, k, v = _qkv(1, 2, 2, 512, 64, seed=4, dtype=torch.float32)
    spec = tkt.SparseSpec(budget=1.0, block_q=64, block_kv=32)
    assert tkt.nsa_select(to_dev(q), to_dev(k), spec) is None
    rep = run_case(q, k, v, spec, False, where="dense")  # attention with selection None
    say(f"  {rep}")


def test_short_sequence_single_tile():
    """S below one block: a single partial tile; forced selection keeps the diagonal only."""
    say("short sequence")
    q, k, v = _qkv(1, 2, 2, 50, 128, seed=6, dtype=torch.bfloat16)
    spec = tkt.SparseSpec(budget=0.3, block_q=128, block_kv=64)
    assert tkt.nsa_select(to_dev(q), to_dev(k), spec) is None  # no candidates: dense
    rep = run_case(q, k, v, tkt.SparseSpec(budget=0.3, force=True), True, where="short")
    say(f"  {rep}")


def test_empty_sequence():
    say("empty sequence")
    q = torch.zeros(1, 2, 0, 64, device="cuda:0")
    spec = tkt.SparseSpec(budget=0.3, force=True)
    sel = tkt.nsa_select(q, q, spec)
    assert sel is not None and sel.keep.numel() == 0 and sel.nnz == 0
    out, lse = tkt.nsa_block_sparse_attn(q, q, q, sel, True)
    assert out.numel() == 0 and lse.numel() == 0
    assert tkt.nsa_select(q, q, tkt.SparseSpec(budget=0.3)) is None


@pytest.mark.parametrize("causal", [False, True])
def test_growing_logits_move_the_softmax_reference(causal):
    """Keys whose scale grows along the sequence make later tiles' logits dominate,
    so the running softmax reference moves on many tiles (online rescale path).
    Outputs reach |O| > 4, where half a bf16 ulp is 0.0156, so the error is
    measured relative to max(1, |O|); a misordered rescale gives O(1) errors."""
    say(f"growing logits causal={causal}")
    B, H, S, D = 1, 4, 4096, 128
    q, k, v = _qkv(B, H, H, S, D, seed=31, dtype=torch.float32)
    ramp = (1.0 + torch.arange(S, dtype=torch.float32) / 256.0)[None, None, :, None]
    k = (k * ramp).to(torch.bfloat16)
    q, v = q.to(torch.bfloat16), v.to(torch.bfloat16)
    rep = run_case(q, k, v, tkt.SparseSpec(budget=0.5), causal, where="growing", relative=True)
    say(f"  {rep}")


@pytest.mark.parametrize("causal", [False, True])
def test_huge_logits_move_the_reference_by_the_guard(causal):
    """q and k scaled by 16: logits reach thousands of scaled units, so a row's
    exponentials against a stale reference overflow (inf) or pass 2^20, and the
    kernel must take the row maximum and recompute those tiles; any slip gives
    inf / NaN or O(1) errors. Softmax rows are nearly one-hot here."""
    say(f"huge logits causal={causal}")
    B, H, S, D = 1, 2, 2048, 128
    q, k, v = _qkv(B, H, H, S, D, seed=37, dtype=torch.float32)
    q, k, v = (q * 16).to(torch.bfloat16), (k * 16).to(torch.bfloat16), v.to(torch.bfloat16)
    rep = run_case(q, k, v, tkt.SparseSpec(budget=0.5), causal, where="huge", relative=True)
    say(f"  {rep}")


@pytest.mark.parametrize("H,S", [(2, 2048), (16, 16384)])
def test_all_tied_scores_pick_lowest_index(H, S):
    """q = 0: every score is +-0, so each row keeps its k_r lowest-index candidates
    (the second case has more than 1024 rows: one wavefront per row)."""
    say(f"all ties H={H} S={S}")
    B, D = 1, 128
    _, k, v = _qkv(B, H, H, S, D, seed=8, dtype=torch.bfloat16)
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16)
    rows = None if S <= 2048 else [(0, 0, 0), (0, H - 1, S // 128 - 1), (0, 3, 40)]
    rep = run_case(q, k, v, tkt.SparseSpec(budget=0.3), False, rows=rows, where="ties")
    say(f"  {rep}")


@pytest.mark.parametrize("nk", [256, 2048])
def test_crowded_threshold_bucket(nk):
    """Five kv tiles score a thousand times above the rest and the rest spread
    over +-10%: the first histogram puts every other candidate into its lowest
    bucket, so the search narrows to that bucket's own value range before
    cutting. Scores are sums of positive terms (no cancellation), so fp32
    rounding on either side stays far below the gaps between them."""
    say(f"crowded bucket nk={nk}")
    B, Hq, Hkv, D, bq, bkv = 1, 16, 4, 64, 64, 16
    S = nk * bkv
    g = torch.Generator().manual_seed(nk)
    q = torch.randn(B, Hq, S, D, generator=g).abs()
    base = torch.randn(1, Hkv, 1, D, generator=g).abs() + 0.5
    f = 0.9 + 0.2 * torch.rand(nk, generator=g)                     # one factor per kv tile
    f[torch.randperm(nk, generator=g)[:5]] = 1000.0
    k = base * f.repeat_interleave(bkv)[None, None, :, None]
    q = q.to(torch.bfloat16)
    k = k.to(torch.bfloat16)
    spec = tkt.SparseSpec(budget=0.1, block_q=bq, block_kv=bkv)
    ref = oracle.select_blocks(q, k, spec.budget, bq, bkv, False, False)
    sel = tkt.nsa_select(to_dev(q), to_dev(k), spec)
    torch.cuda.synchronize()
    _, nflag = check_selection(sel, ref, "crowded")
    say(f"  rows {B * Hq * (S // bq)}, near-tie rows {nflag}")


def test_few_long_rows():
    """Few selection rows (a workgroup per row) with 4096 kv tiles each, pins
    and drops, against the oracle; attention on sampled rows."""
    say("few long rows")
    B, Hq, Hkv, S, D = 1, 2, 1, 65536, 64
    q, k, v = _qkv(B, Hq, Hkv, S, D, seed=19, dtype=torch.bfloat16)
    spec = tkt.SparseSpec(budget=0.05, block_q=1024, block_kv=16)
    nq, nk = S // 1024, S // 16
    rng = np.random.default_rng(19)
    pins = (rng.random((1, 1, nq, nk)) < 0.01).astype(np.int8)
    drops = (rng.random((1, Hq, nq, nk)) < 0.02).astype(np.int8)
    rep = run_case(q, k, v, spec, True, pins=pins, drops=drops, rows=[(0, 0, 5), (0, 1, 63)], where="few long rows")
    say(f"  {rep}")


@pytest.mark.parametrize("S,bq,bkv,Hq", [(16384, 256, 16, 2), (8192, 128, 32, 2), (8192, 256, 16, 2),
                                         # more than 1024 rows: one wavefront per row
                                         (8192, 64, 16, 16), (32768, 256, 16, 16), (4096, 32, 64, 24),
                                         (6000, 64, 24, 12)])
def test_exact_ties_take_lowest_index(S, bq, bkv, Hq):
    """Every kv tile repeats one of three key vectors, so pooled keys are exact
    copies and a row's scores fall into three groups of exactly equal values,
    well apart from each other. The boundary group must be cut at the lowest
    kv indices (score descending, index ascending): the expected keep is built
    from float64 group scores and compared bit for bit, pins and drops
    included."""
    say(f"exact ties S={S} bq={bq} bkv={bkv} Hq={Hq}")
    B, Hkv, D = 1, 1, 64
    g = torch.Generator().manual_seed(S + bq)
    q = torch.randn(B, Hq, S, D, generator=g).to(torch.bfloat16)
    V = torch.randn(3, D, generator=g).to(torch.bfloat16)
    nq, nk = -(-S // bq), -(-S // bkv)
    tile_of = torch.arange(S) // bkv
    k = V[tile_of % 3].reshape(1, 1, S, D).contiguous()
    rng = np.random.default_rng(S)
    pins = (rng.random((1, 1, nq, nk)) < 0.02).astype(np.int8)
    drops = (rng.random((1, Hq, nq, nk)) < 0.05).astype(np.int8)
    budget = 0.2
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv)
    sel = tkt.nsa_select(to_dev(q), to_dev(k), spec, pins, drops)
    torch.cuda.synchronize()
    got = sel.keep.cpu().numpy() != 0
    pq = oracle.pool_blocks(q, bq).double().numpy()                    # (B, Hq, NQ, D)
    # the last kv tile may be ragged: its pooled key is still one of the three vectors
    gs = pq @ V.double().numpy().T                                     # (B, Hq, NQ, 3) group scores
    gap = np.sort(gs, -1)
    # Rows whose three group scores are far apart next to fp32 rounding of a
    # pooled score (~(bq + D) 2^-24 relative) have one exact answer; the rare
    # rows with two close groups are held to the selection rules only.
    exact = np.all(np.diff(gap, axis=-1) > 1e-4 * np.abs(gap).max(axis=-1, keepdims=True), axis=-1)
    assert exact.mean() > 0.9
    plan = oracle.selection_plan(nq, nk, bq, bkv, budget, B, Hq, pins, drops)
    want = plan["must"] & ~plan["forbidden"]
    grp = np.arange(nk) % 3
    for h in range(Hq):
        for i in range(nq):
            cand = np.nonzero(plan["candidates"][0, h, i])[0]
            order = sorted(cand, key=lambda j: (-gs[0, h, i, grp[j]], j))
            want[0, h, i, order[:int(plan["k"][0, h, i])]] = True
    assert np.array_equal(got[exact], want[exact])
    must = plan["must"] & ~plan["forbidden"]
    assert np.all(got[must]) and not np.any(got & plan["forbidden"])
    assert np.array_equal(got.sum(-1), want.sum(-1))
    r_ptr, r_col = oracle.keep_to_csr(got.astype(np.int8))
    assert np.array_equal(sel.row_ptr.cpu().numpy(), r_ptr) and np.array_equal(sel.col_idx.cpu().numpy(), r_col)
    assert np.array_equal(r_ptr, oracle.keep_to_csr(want.astype(np.int8))[0])


@pytest.mark.parametrize("B,Hq,Hkv,S,bq,bkv,budget", [
    (2, 16, 4, 8192, 128, 64, 0.25),     # 128 kv tiles
    (1, 24, 8, 16384, 128, 16, 0.05),    # 1024 kv tiles
    (1, 16, 4, 32768, 256, 16, 0.05),    # 2048 kv tiles
    (1, 16, 16, 8000, 64, 64, 0.30),     # 125 kv tiles (not a multiple of 4)
    (1, 12, 3, 6100, 64, 16, 0.10),      # 382 kv tiles, ragged tail
    (1, 16, 4, 8000, 64, 16, 0.10),      # 500 kv tiles: a multiple of 4, second group of 256 ragged
    (1, 8, 2, 20800, 128, 16, 0.97),     # 1300 kv tiles, budget near 1: the cut in the lowest buckets
    (1, 16, 4, 4096, 32, 16, 0.98),      # 256 kv tiles, all but a few candidates kept
])
def test_many_rows_pins_drops(B, Hq, Hkv, S, bq, bkv, budget):
    """More than 1024 selection rows (one wavefront per row) against the oracle,
    with per-batch pins and per-head drops covering diagonal tiles too."""
    say(f"many rows B={B} Hq={Hq} S={S} bq={bq} bkv={bkv}")
    D = 64
    q, k, _ = _qkv(B, Hq, Hkv, S, D, seed=S + Hq, dtype=torch.bfloat16)
    nq, nk = -(-S // bq), -(-S // bkv)
    rng = np.random.default_rng(S)
    pins = (rng.random((B, 1, nq, nk)) < 0.02).astype(np.int8)
    drops = (rng.random((1, Hq, nq, nk)) < 0.03).astype(np.int8)
    spec = tkt.SparseSpec(budget=budget, block_q=bq, block_kv=bkv)
    ref = oracle.select_blocks(q, k, budget, bq, bkv, False, False, pins, drops)
    sel = tkt.nsa_select(to_dev(q), to_dev(k), spec, pins, drops)
    torch.cuda.synchronize()
    _, nflag = check_selection(sel, ref, "many rows")
    say(f"  rows {B * Hq * nq}, near-tie rows {nflag}, nnz {sel.nnz}")


def test_widest_row_nk4096():
    """NK = 4096 (64 score slots per lane), per-head GQA scoring, sampled attention rows."""
    say("nk4096")
    B, Hq, Hkv, S, D = 1, 2, 1, 4096 * 16, 64
    q, k, v = _qkv(B, Hq, Hkv, S, D, seed=9, dtype=torch.bfloat16)
    spec = tkt.SparseSpec(budget=0.02, block_q=64, block_kv=16)
    rows = [(0, 0, 0), (0, 1, 517), (0, 0, 1023)]
    rep = run_case(q, k, v, spec, True, rows=rows, where="nk4096")
    say(f"  {rep}")


def test_error_codes_do_not_launch():
    say("error codes")
    q = torch.zeros(1, 4, 128, 128, dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros(1, 3, 128, 128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(tkt.NsaError) as e:
        tkt.nsa_select(q, k, tkt.SparseSpec())
    assert e.value.status == -2
    with pytest.raises(tkt.NsaError) as e:
        tkt.nsa_select(q, q, tkt.SparseSpec(budget=float("nan")))
    assert e.value.status == -6
    with pytest.raises(tkt.NsaError) as e:
        tkt.nsa_block_sparse_attn(q, q.float(), q, None, True)
    assert e.value.status == -3
