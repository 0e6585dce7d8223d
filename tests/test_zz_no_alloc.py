"""The allocation-free decode attention (nsa_decode_attn_static, split
partials in the library's static device buffer) against nsa_decode_attn with
a caller workspace, through the C ABI: two calls in a row, the second on a
smaller request, so the second reads a buffer the first left behind."""
import numpy as np
import pytest
import torch

import top_kv_tile_amd as tkt
from parity_util import say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, n, length, cap, D, seed, select):
    g = torch.Generator().manual_seed(seed)
    kc, vc = (torch.randn(B, Hkv, cap, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, n, D, generator=g).to(torch.bfloat16)
    kd, vd, qd = to_dev(kc), to_dev(vc), to_dev(q)
    sel = None
    if select:
        pooled = torch.zeros(B, Hkv, cap // 64, D, dtype=torch.float32, device="cuda:0")
        tkt.nsa_decode_pool_update(kd, 0, length, 64, pooled)
        spec = tkt.SparseSpec(budget=0.05, block_q=32, block_kv=64, force=True)
        nk = -(-length // 64)
        pins = np.zeros((1, 1, 1, nk), np.int8)
        pins[..., 0] = 1
        sel = tkt.nsa_decode_select(qd, pooled, length, length - n, spec, pins)
    return qd, kd, vd, sel


@pytest.mark.parametrize("first,second", [
    # (B, Hq, Hkv, n, length, cap, D, seed, select): a 128k decoding step, then a shorter one
    ((1, 64, 8, 1, 131072, 131072, 128, 1, True), (1, 16, 4, 1, 20000, 32768, 128, 2, True)),
    ((2, 8, 2, 4, 16000, 16384, 128, 3, False), (1, 4, 4, 3, 5000, 8192, 64, 4, False)),
])
def test_static_matches_workspace_call(first, second):
    for case in (first, second):
        say(f"static decode {case}")
        B, Hq, Hkv, n, length, cap, D, seed, select = case
        qd, kd, vd, sel = _case(*case)
        ws = torch.empty(1, dtype=torch.uint8, device="cuda:0")
        ref_o, ref_l = tkt.nsa_decode_attn(qd, kd, vd, length, length - n, sel, workspace=ws)
        out = torch.full_like(qd, float("nan"))
        lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda:0")
        tkt.nsa_decode_attn_static(qd, kd, vd, length, length - n, sel, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"{case}: output differs from the workspace call"
        assert torch.equal(lse, ref_l), f"{case}: lse differs from the workspace call"
        need = tkt.nsa_decode_attn_workspace_size(qd, kd, length, length - n, sel)
        assert 0 < need <= 16 << 20, need          # the static buffer was used, within its size
        say(f"  equal; split partials {need} bytes")
