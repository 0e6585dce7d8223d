"""Seeded random sweep of the pooled score product with more than 64 query
tiles per selection head (the split-operand bf16 kernel) against the oracle:
random head dims, tile sizes, GQA ratios, head_shared scoring, input dtypes
and magnitudes, with ragged query and kv tiles (block counts with and without
the XCD numbering). Every score must lie within the fp32 bound of the
oracle's, 4 D 2^-24 sum_d |q_d k_d| (both sides round an fp32 dot product).

The reading followed is the selector.py page's score_blocks: the raw dot
product of the fp32 pooled query and key tiles (head means when head_shared)."""
import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from parity_util import say, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 12


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128, 256]))
    bq = int(rng.choice([32, 64, 128]))
    bkv = int(rng.choice([16, 32, 64]))
    nq = int(rng.integers(65, 400))
    S = nq * bq - int(rng.integers(0, bq))  # ragged last query tile
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    return dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, S=S, D=D, bq=bq, bkv=bkv,
                shared=bool(rng.integers(0, 4) == 0), f32=bool(rng.integers(0, 2)),
                scale=float(2.0 ** rng.integers(-6, 7)))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_scores(seed):
    c = _case(seed)
    say(f"random scores {c}")
    g = torch.Generator().manual_seed(7000 + seed)
    dt = torch.float32 if c["f32"] else torch.bfloat16
    q = (torch.randn(c["B"], c["Hq"], c["S"], c["D"], generator=g) * c["scale"]).to(dt)
    k = torch.randn(c["B"], c["Hkv"], c["S"], c["D"], generator=g).to(dt)
    spec = tkt.SparseSpec(block_q=c["bq"], block_kv=c["bkv"], head_shared=c["shared"])
    got = tkt.nsa_score_blocks(to_dev(q), to_dev(k), spec).cpu().numpy().astype(np.float64)
    ref = oracle.score_blocks(q, k, c["bq"], c["bkv"], c["shared"]).astype(np.float64)
    qh, kh = oracle.head_operands(oracle.pool_blocks(q, c["bq"]), oracle.pool_blocks(k, c["bkv"]), c["shared"])
    mag = np.abs(qh.double().numpy()) @ np.swapaxes(np.abs(kh.double().numpy()), -1, -2)
    assert got.shape == ref.shape and got.shape[2] > 64
    err = np.abs(got - ref)
    bound = 4 * c["D"] * 2.0 ** -24 * mag + 1e-30
    assert np.all(err <= bound), f"worst error / bound {float((err / bound).max()):.3g}"
    say(f"  max error / bound {float((err / bound).max()):.3g}")
