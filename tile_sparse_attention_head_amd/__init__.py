"""Tile-sparse self-attention for video DiTs on MI355X (gfx950).

The hot path of "Veda: Scalable Video Diffusion via Distilled Sparse
Attention" -- head-aware tile permutation, TripPool tile scoring, top-k tile
selection, tile-skipping attention and the max-pooled attention map -- as
hand-written HIP kernels behind the C ABI in include/veda.h (libveda.so).
This package is the thin Python binding (``_lib``) plus a layer object that
owns buffers and issues the calls in order (``layer``).
"""
from ._lib import (  # noqa: F401
    LIB_PATH, VEDA_BF16, VEDA_F32, VEDA_FWD, VEDA_FWD_T, VEDA_INV, VedaError, csr_nnz, lib,
    veda_distill_grad, veda_distill_grad_noalloc, veda_distill_grad_workspace, veda_head_choose,
    veda_head_sq_error, veda_head_sq_error_workspace, veda_sparse_attn_bwd, veda_sparse_attn_bwd_tiles,
    veda_sparse_attn_bwd_workspace, status_string, tiles_numel, tokens_numel, veda_keep_count, veda_layout, veda_layout_init,
    veda_oracle_maxpool_map, veda_oracle_maxpool_map_workspace, veda_score_select, veda_select_tiles,
    veda_sparse_attn_fwd, veda_sparse_attn_fwd_tokens, veda_sparse_attn_fwd_workspace,
    veda_tile_permute, veda_tile_permute_pool,
    veda_tile_score, veda_tripool_score)
from .layer import TileSparseAttention  # noqa: F401
from .tiling_search import search_tile_shapes  # noqa: F401
