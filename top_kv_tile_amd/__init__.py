"""MI355X (gfx950) block-sparse attention driven by top-k KV-tile selection.

The work runs in hand-written HIP kernels behind the C ABI of include/nsa.h
(``libnsa.so``, built in-tree by ``python -m top_kv_tile_amd.build``); this
package is its thin Python binding. See ``top_kv_tile_amd.nsa``.
"""
from .nsa import (  # noqa: F401
    EXPORTS,
    NSA_CURVE_HILBERT,
    NSA_CURVE_MORTON,
    LIB_PATH,
    NsaError,
    Plan,
    Selection,
    Sizes,
    SparseSpec,
    lib,
    nsa_attn_bwd_workspace_size,
    nsa_block_sparse_attn,
    nsa_block_sparse_attn_bwd,
    nsa_curve_order,
    nsa_decode_attn,
    nsa_decode_attn_static,
    nsa_decode_attn_workspace_size,
    nsa_decode_pool_update,
    nsa_decode_select,
    nsa_permute_tokens,
    nsa_plan_cache_clear,
    nsa_plan_cache_config,
    nsa_plan_cache_stats,
    nsa_plan_create,
    nsa_pool_blocks,
    nsa_radial_blocks,
    nsa_schedule,
    nsa_score_blocks,
    nsa_select,
    nsa_select_planned,
    nsa_select_sizes,
    nsa_selection_density,
    nsa_stage_timing_begin,
    nsa_stage_timing_end,
    nsa_status_string,
)

__version__ = "0.1.0"
