"""GPU parity of decoding over a KV cache: the incrementally updated pooled
keys, the decode selection and the decode attention, step by step as the cache
grows, against the decode oracle (fresh pooling, select_blocks at the queries'
absolute positions, causal attention in absolute positions)."""
import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from parity_util import check_attention, check_selection, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,Hq,Hkv,D,bq,shared", [(torch.bfloat16, 8, 2, 128, 128, False),
                                                      (torch.bfloat16, 4, 4, 64, 32, True),
                                                      (torch.bfloat16, 8, 4, 128, 64, True),
                                                      (torch.float32, 4, 2, 64, 64, False)])
def test_decode_loop(dtype, Hq, Hkv, D, bq, shared):
    say(f"decode loop {dtype} Hq={Hq} Hkv={Hkv} D={D} bq={bq} shared={shared}")
    B, cap, bkv = 1, 2048, 64
    g = torch.Generator().manual_seed(Hq * D + bq)
    kc = torch.randn(B, Hkv, cap, D, generator=g).to(dtype)
    vc = torch.randn(B, Hkv, cap, D, generator=g).to(dtype)
    qs = torch.randn(B, Hq, cap, D, generator=g).to(dtype)
    kd, vd = to_dev(kc), to_dev(vc)
    pooled = torch.zeros(B, Hkv, cap // bkv, D, dtype=torch.float32, device="cuda:0")
    spec = tkt.SparseSpec(budget=0.3, block_q=bq, block_kv=bkv, head_shared=shared, force=True)
    length = 0
    for step, n in enumerate([1000, 1, 1, 5, 1, 70, 1]):  # a prefill, then single tokens and chunks
        old, length = length, length + n
        tkt.nsa_decode_pool_update(kd, old, length, bkv, pooled)
        torch.cuda.synchronize()
        ref_pool = oracle.decode_pool(kc, length, bkv)
        got_pool = pooled[:, :, :ref_pool.shape[2]].cpu()
        assert (got_pool - ref_pool).abs().max().item() <= 2 * bkv * 2.0 ** -24 * kc.float().abs().max().item()
        pos0 = length - n
        q = qs[:, :, pos0:length].contiguous()
        qd = to_dev(q)
        sel = tkt.nsa_decode_select(qd, pooled, length, pos0, spec)
        ref = oracle.decode_select(q, kc, length, pos0, spec.budget, bq, bkv, shared, True)
        keep, _ = check_selection(sel, ref, f"step {step}")
        out, lse = tkt.nsa_decode_attn(qd, kd, vd, length, pos0, sel)
        ref_o, ref_l = oracle.decode_attention(q, kc, vc, length, pos0, keep, bq, bkv)
        check_attention(out, lse, ref_o, ref_l, "bf16" if dtype == torch.bfloat16 else "f32",
                        where=f"decode step {step}")


def test_dense_decode_attention():
    say("dense decode")
    B, Hq, Hkv, cap, D = 2, 8, 2, 1536, 128
    g = torch.Generator().manual_seed(4)
    kc, vc = (torch.randn(B, Hkv, cap, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, 3, D, generator=g).to(torch.bfloat16)
    length = 1201
    out, lse = tkt.nsa_decode_attn(to_dev(q), to_dev(kc), to_dev(vc), length, length - 3, None)
    nk = -(-length // 64)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, length, length - 3, np.ones((1, 1, 1, nk), np.int8), 32, 64)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="dense decode")


@pytest.mark.parametrize("n,shared", [(1, False), (4, False), (3, True)])
def test_split_decode_attention(n, shared):
    """Few query rows over a long cache: each row's tiles are split over several
    workgroups and merged. A head whose tiles are all dropped (empty row), a
    ragged last tile, and splits that get no tile."""
    say(f"split decode n={n} shared={shared}")
    B, Hq, Hkv, cap, D, bq, bkv = 2, 8, 2, 16384, 128, 32, 64
    length = 15990
    g = torch.Generator().manual_seed(31 + n)
    kc, vc = (torch.randn(B, Hkv, cap, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, n, D, generator=g).to(torch.bfloat16)
    pos0 = length - n
    nk = -(-length // bkv)
    kd, vd = to_dev(kc), to_dev(vc)
    pooled = torch.zeros(B, Hkv, cap // bkv, D, dtype=torch.float32, device="cuda:0")
    tkt.nsa_decode_pool_update(kd, 0, length, bkv, pooled)
    rng = np.random.default_rng(n)
    pins = (rng.random((B, 1, 1, nk)) < 0.05).astype(np.int8)
    drops = np.zeros((1, 1 if shared else Hq, 1, nk), np.int8)
    if not shared:
        drops[0, 5] = 1  # every tile of head 5: its rows are empty
    spec = tkt.SparseSpec(budget=0.25, block_q=bq, block_kv=bkv, head_shared=shared, force=True)
    qd = to_dev(q)
    sel = tkt.nsa_decode_select(qd, pooled, length, pos0, spec, pins=pins, drops=drops)
    ref = oracle.decode_select(q, kc, length, pos0, spec.budget, bq, bkv, shared, True, pins=pins, drops=drops)
    keep, _ = check_selection(sel, ref, "split select")
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, length, pos0, sel)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, length, pos0, keep, bq, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="split decode")
    if not shared:
        assert torch.isneginf(lse[:, 5]).all() and (out[:, 5] == 0).all()
    # dense over the same cache
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, length, pos0, None)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, length, pos0, np.ones((1, 1, 1, nk), np.int8), bq, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="split dense decode")


@pytest.mark.parametrize("Hq,Hkv,D,n,bq", [(8, 2, 128, 40, 64), (16, 2, 64, 9, 32), (6, 3, 128, 1, 32)])
def test_packed_gqa_decode(Hq, Hkv, D, n, bq):
    """A selection shared by the heads (or none): the heads of a GQA group are
    packed into one workgroup's rows. 40 tokens x 4 heads span two packed
    tiles; causal masks inside the new tokens; split partials on long rows."""
    say(f"packed decode Hq={Hq} Hkv={Hkv} D={D} n={n}")
    B, cap, bkv = 2, 4096, 64
    length = 3001 + n
    g = torch.Generator().manual_seed(Hq * 100 + n)
    kc, vc = (torch.randn(B, Hkv, cap, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, n, D, generator=g).to(torch.bfloat16)
    pos0 = length - n
    nk = -(-length // bkv)
    kd, vd, qd = to_dev(kc), to_dev(vc), to_dev(q)
    pooled = torch.zeros(B, Hkv, cap // bkv, D, dtype=torch.float32, device="cuda:0")
    tkt.nsa_decode_pool_update(kd, 0, length, bkv, pooled)
    spec = tkt.SparseSpec(budget=0.2, block_q=bq, block_kv=bkv, head_shared=True, force=True)
    sel = tkt.nsa_decode_select(qd, pooled, length, pos0, spec)
    ref = oracle.decode_select(q, kc, length, pos0, spec.budget, bq, bkv, True, True)
    keep, _ = check_selection(sel, ref, "packed select")
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, length, pos0, sel)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, length, pos0, keep, bq, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="packed decode")
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, length, pos0, None)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, length, pos0, np.ones((1, 1, 1, nk), np.int8), bq, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="packed dense decode")


@pytest.mark.parametrize("shared", [False, True])
def test_decode_128k_cache(shared):
    """The decoding step bench.py times, at its size: one new token over a
    131 072-token cache, 64 query heads over 8 kv heads, per-head or shared
    selection with the sink tile pinned; every head against the oracle, and
    the dense call too."""
    say(f"decode 128k shared={shared}")
    B, Hq, Hkv, L, D, bkv = 1, 64, 8, 131072, 128, 64
    g = torch.Generator().manual_seed(77 + shared)
    kc, vc = (torch.randn(B, Hkv, L, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, 1, D, generator=g).to(torch.bfloat16)
    nk = L // bkv
    kd, vd, qd = to_dev(kc), to_dev(vc), to_dev(q)
    pooled = torch.zeros(B, Hkv, nk, D, dtype=torch.float32, device="cuda:0")
    tkt.nsa_decode_pool_update(kd, 0, L - 1, bkv, pooled)
    tkt.nsa_decode_pool_update(kd, L - 1, L, bkv, pooled)  # the step's own token
    pins = np.zeros((1, 1, 1, nk), np.int8)
    pins[..., 0] = 1
    spec = tkt.SparseSpec(budget=0.05, block_q=32, block_kv=bkv, head_shared=shared)
    sel = tkt.nsa_decode_select(qd, pooled, L, L - 1, spec, pins=pins)
    ref = oracle.decode_select(q, kc, L, L - 1, spec.budget, 32, bkv, shared, False, pins=pins)
    keep, _ = check_selection(sel, ref, "128k select")
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, L, L - 1, sel)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, L, L - 1, keep, 32, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="128k decode")
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, L, L - 1, None)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, L, L - 1, np.ones((1, 1, 1, nk), np.int8), 32, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="128k dense decode")


@pytest.mark.parametrize("n,pin_rows,drop_rows", [(1, 1, 1), (3, 1, 1), (1, 0, 1), (1, 2, 1), (2, 1, 16)])
def test_decode_mask_rows(n, pin_rows, drop_rows):
    """Decode selection with pin and drop masks of one row shared by every row
    (carried in the top-k launch: nothing is uploaded), of several rows (copied
    to the device), or absent, for one and for a few new tokens."""
    say(f"decode masks n={n} pin_rows={pin_rows} drop_rows={drop_rows}")
    B, Hq, Hkv, L, D, bkv, bq = 2, 16, 4, 8192, 128, 64, 32
    g = torch.Generator().manual_seed(1000 + 10 * n + pin_rows + drop_rows)
    kc, vc = (torch.randn(B, Hkv, L, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, n, D, generator=g).to(torch.bfloat16)
    nk = L // bkv
    rng = np.random.default_rng(n + pin_rows + drop_rows)
    pins = None
    if pin_rows:
        pins = (rng.random((pin_rows, 1, 1, nk)) < 0.03).astype(np.int8)
        pins[..., 0] = 1
        pins[..., nk // 2] = 1
    drops = (rng.random((1, drop_rows, 1, nk)) < 0.1).astype(np.int8)
    drops[..., nk // 2] = 1  # pinned and dropped: the drop wins
    kd, vd, qd = to_dev(kc), to_dev(vc), to_dev(q)
    pooled = torch.zeros(B, Hkv, nk, D, dtype=torch.float32, device="cuda:0")
    tkt.nsa_decode_pool_update(kd, 0, L, bkv, pooled)
    spec = tkt.SparseSpec(budget=0.1, block_q=bq, block_kv=bkv, head_shared=False)
    sel = tkt.nsa_decode_select(qd, pooled, L, L - n, spec, pins=pins, drops=drops)
    ref = oracle.decode_select(q, kc, L, L - n, spec.budget, bq, bkv, False, False, pins=pins, drops=drops)
    keep, _ = check_selection(sel, ref, "mask rows select")
    out, lse = tkt.nsa_decode_attn(qd, kd, vd, L, L - n, sel)
    ref_o, ref_l = oracle.decode_attention(q, kc, vc, L, L - n, keep, bq, bkv)
    check_attention(out, lse, ref_o, ref_l, "bf16", where="mask rows decode")
