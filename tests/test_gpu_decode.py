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
