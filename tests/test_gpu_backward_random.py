"""Seeded random sweep of the attention gradients against the fp64 gradient
oracle, on the GPU's own selection, with the bounds of test_gpu_backward.py:
random GQA shapes (groups of 1 to 8), D 64 / 128, query tiles of 32 to 128
tokens, causal or not, per-head or shared scoring, ragged S, budgets, and pins
and drops on or off (a dropped diagonal tile leaves rows with no key). Every
element of dq, dk and dv is compared."""
import numpy as np
import pytest
import torch

import top_kv_tile_amd as tkt
from parity_util import say
from test_gpu_backward import _inputs, run_bwd_case

pytestmark = pytest.mark.gpu

N_CASES = 12


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128]))
    bq = int(rng.choice([32, 64, 96, 128]))
    S = int(rng.integers(bq + 1, 2048))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    return dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, S=S, D=D, bq=bq, causal=bool(rng.integers(0, 2)),
                shared=bool(rng.random() < 0.25), budget=float(rng.uniform(0.05, 0.6)),
                pins=bool(rng.integers(0, 2)), drops=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_backward(seed):
    c = _case(seed)
    say(f"random backward {c}")
    B, Hq, Hkv, S, D, bq = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["bq"]
    q, k, v, do = _inputs(B, Hq, Hkv, S, D, seed=7000 + seed, dtype=torch.bfloat16)
    nq, nk = -(-S // bq), -(-S // 64)
    Hs = 1 if c["shared"] else Hq
    rng = np.random.default_rng(seed)
    pins = (rng.random((B, 1, nq, nk)) < 0.03).astype(np.int8) if c["pins"] else None
    drops = (rng.random((1, Hs, nq, nk)) < 0.05).astype(np.int8) if c["drops"] else None
    spec = tkt.SparseSpec(budget=c["budget"], block_q=bq, block_kv=64, head_shared=c["shared"])
    rep = run_bwd_case(q, k, v, do, spec, c["causal"], pins=pins, drops=drops, where=f"random backward {seed}")
    say(f"  {rep}")
