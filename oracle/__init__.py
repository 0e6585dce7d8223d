"""CPU oracle for top-k KV-tile selection and block-sparse attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``top_kv_tile_amd``) and never takes an input or an expected value
from it.

The oracle is plain and slow on purpose: each function is the written-out
definition of one step of the method, citing the page it follows.

Pages:
  * ``selector.py`` -- the page "automatic/modules/attention/sparse/selector.py"
    (module docstring: fixed-budget block selection).
  * "todo" -- native-sparse-attention-pytorch issue #1.
  * "Arbitrary masks" -- NATTEN issue 124.
  * "Doubts about Flex Attention masks used" -- native-sparse-attention-pytorch
    discussion #8.
  * "Optimal ordering with block mask" -- attention-gym issue 56.
"""
from .select import (  # noqa: F401
    block_count,
    pool_blocks,
    diagonal_blocks,
    head_operands,
    score_blocks,
    selection_plan,
    keep_per_row,
    select_blocks,
    keep_to_csr,
    rank_select,
    NEAR_TIE_REL,
)
from .attention import attention, attention_dense_literal, visible_key_counts  # noqa: F401
from .attention_bwd import attention_backward  # noqa: F401
from .controls import schedule, radial_blocks, density  # noqa: F401
from .reorder import morton_order, hilbert_order, apply_order, undo_order  # noqa: F401
from .decode import decode_pool, decode_select, decode_attention  # noqa: F401
