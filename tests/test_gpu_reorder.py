"""GPU parity of token reordering: nsa_permute_tokens against the oracle's
gather / scatter, bit-exact (it moves bytes), on curve orders of 2D and 3D
grids, with a round trip and untouched rows for out-of-range entries."""
import numpy as np
import pytest
import torch

import oracle
import top_kv_tile_amd as tkt
from parity_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dims,D,curve", [((32, 64), 128, "morton"), ((16, 16, 8), 64, "hilbert"),
                                          ((5, 7), 128, "hilbert"), ((128, 256), 128, "hilbert")])
def test_permute_matches_oracle(dtype, dims, D, curve):
    say(f"permute {dims} D={D} {curve} {dtype}")
    S = int(np.prod(dims))
    kind = tkt.NSA_CURVE_MORTON if curve == "morton" else tkt.NSA_CURVE_HILBERT
    perm = tkt.nsa_curve_order(kind, dims)
    ref_perm = oracle.morton_order(dims) if curve == "morton" else oracle.hilbert_order(dims)
    assert np.array_equal(perm, ref_perm)
    g = torch.Generator().manual_seed(S)
    x = torch.randn(2, 3, S, D, generator=g).to(dtype)
    xd = to_dev(x)
    pd = torch.from_numpy(perm).to("cuda:0")
    y = tkt.nsa_permute_tokens(xd, pd)
    back = tkt.nsa_permute_tokens(y, pd, inverse=True)
    torch.cuda.synchronize()
    want = oracle.apply_order(x.float().numpy(), ref_perm)
    assert np.array_equal(y.float().cpu().numpy(), want)
    assert np.array_equal(back.float().cpu().numpy(), oracle.undo_order(want, ref_perm))
    assert torch.equal(back, xd)


def test_out_of_range_entries_are_skipped():
    say("permute out of range")
    S, D = 64, 128
    perm = np.arange(S, dtype=np.int32)[::-1].copy()
    perm[5] = S + 3
    perm[9] = -1
    x = torch.randn(1, 2, S, D).to(torch.bfloat16)
    y = torch.full_like(x, 7.0).to("cuda:0")
    tkt.nsa_permute_tokens(to_dev(x), torch.from_numpy(perm).to("cuda:0"), out=y)
    yc = y.cpu()
    for m in range(S):
        if m in (5, 9):
            assert bool((yc[:, :, m] == 7.0).all())
        else:
            assert torch.equal(yc[:, :, m], x[:, :, perm[m]])


def test_permute_bandwidth_2gib():
    """(1, 64, 131072, 128) bf16: 2 GiB read and 2 GiB written per call."""
    x = torch.empty(1, 64, 131072, 128, dtype=torch.bfloat16, device="cuda:0").normal_()
    perm = torch.from_numpy(tkt.nsa_curve_order(tkt.NSA_CURVE_HILBERT, (256, 512))).to("cuda:0")
    y = torch.empty_like(x)
    for _ in range(2):
        tkt.nsa_permute_tokens(x, perm, out=y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        tkt.nsa_permute_tokens(x, perm, out=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    gbs = 2 * x.numel() * 2 / (ms * 1e-3) / 1e9
    say(f"  permute 2 GiB: {ms:.3f} ms, {gbs:.0f} GB/s read+write")
    assert torch.equal(y[0, 0, 0], x[0, 0, int(perm[0])])
