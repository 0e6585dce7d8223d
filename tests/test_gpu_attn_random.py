"""Seeded random sweep of selection + block-sparse attention against the oracle
on every row: random GQA shapes, D 64 / 128, query tiles of 32 to 128 tokens,
causal or not, budgets, pins and drops (empty rows included), and logit scales
from 0.25 to 12 (the softmax reference moves by its guard on the larger ones).
Outputs are compared relative to max(1, |O|) (the scaled cases reach |O| > 1),
with the bf16 tolerances of the other parity tests; the LSE within 1e-3."""
import numpy as np
import pytest
import torch

import top_kv_tile_amd as tkt
from parity_util import run_case, say

pytestmark = pytest.mark.gpu

N_CASES = 16


def _case(seed):
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 128]))
    bq = int(rng.choice([32, 64, 96, 128]))
    bkv = 64  # the matrix-core forward takes 64-key tiles
    S = int(rng.integers(bq + 1, 3072))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    return dict(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, bq=bq, bkv=bkv, causal=bool(rng.integers(0, 2)),
                budget=float(rng.uniform(0.05, 0.7)), pins=bool(rng.integers(0, 2)),
                drops=bool(rng.integers(0, 2)), scale=float(rng.choice([0.25, 1.0, 4.0, 12.0])))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_attention(seed):
    c = _case(seed)
    say(f"random attention {c}")
    B, Hq, Hkv, S, D, bq, bkv = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["bq"], c["bkv"]
    g = torch.Generator().manual_seed(9000 + seed)
    q = (torch.randn(B, Hq, S, D, generator=g) * c["scale"] ** 0.5).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, S, D, generator=g) * c["scale"] ** 0.5).to(torch.bfloat16)
    v = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    nq, nk = -(-S // bq), -(-S // bkv)
    rng = np.random.default_rng(seed)
    pins = (rng.random((B, 1, nq, nk)) < 0.03).astype(np.int8) if c["pins"] else None
    drops = (rng.random((1, Hq, nq, nk)) < 0.05).astype(np.int8) if c["drops"] else None
    spec = tkt.SparseSpec(budget=c["budget"], block_q=bq, block_kv=bkv)
    rep = run_case(q, k, v, spec, c["causal"], pins, drops, where=f"random attention {seed}", relative=True)
    say(f"  {rep}")
