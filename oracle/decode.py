"""Oracle for decode-time selection and attention over a growing KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Decoding is among the inference pathways listed on "todo"
(native-sparse-attention-pytorch issue #1: KV-cache management, computing the
importance score and loading only the selected KV blocks, a running pooled key
sequence, any sequence length). The selection page defines the selection for
one query and one key sequence aligned at position 0; for decoding, the new
query tokens sit at the end of the cache. The reading taken here: n query
tokens at absolute positions q_pos0 .. q_pos0 + n - 1 against the first L
cached keys (q_pos0 + n <= L):

* the pooled keys are the page's pool_blocks of the L cached tokens (a partly
  filled last tile is averaged over its real length);
* the query tokens are pooled in tiles of block_q counted from q_pos0, and
  everything else is select_blocks with the diagonal measured at the queries'
  absolute positions;
* attention is causal in absolute positions: key u is visible to query t iff
  its tile is kept and u <= q_pos0 + t.
"""
from __future__ import annotations

import torch

from .attention import attention
from .select import pool_blocks, select_blocks

__all__ = ["decode_pool", "decode_select", "decode_attention"]


def decode_pool(k_cache: torch.Tensor, length: int, block_kv: int) -> torch.Tensor:
    """Pooled keys of the first `length` cached tokens, fp32 (B, Hkv, ceil(length / block_kv), D)."""
    return pool_blocks(k_cache[..., :length, :], block_kv)


def decode_select(q: torch.Tensor, k_cache: torch.Tensor, length: int, q_pos0: int, budget: float,
                  block_q: int, block_kv: int, head_shared: bool = False, force: bool = False,
                  pins=None, drops=None):
    """select_blocks for the new query tokens against the cache (see the module docstring)."""
    if q_pos0 < 0 or q_pos0 + q.shape[-2] > length:
        raise ValueError("the query tokens must lie inside the cache")
    return select_blocks(q, k_cache[..., :length, :], budget, block_q, block_kv, head_shared, force,
                         pins, drops, q_offset=q_pos0)


def decode_attention(q, k_cache, v_cache, length: int, q_pos0: int, keep, block_q: int, block_kv: int,
                     rows=None):
    """Causal attention of the new query tokens over the kept tiles of the cache, fp64."""
    return attention(q, k_cache[..., :length, :], v_cache[..., :length, :], keep, block_q, block_kv, True,
                     rows=rows, q_offset=q_pos0)
