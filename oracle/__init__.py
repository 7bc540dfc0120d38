"""Plain fp64 CPU oracle for the tile-sparse attention path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the HIP kernels are checked against.  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path (the C-ABI library and its Python binding) never does, and this package
imports nothing from the product path.

Citations: "Veda §x" is the technical summary of "Veda: Scalable Video
Diffusion via Distilled Sparse Attention" on gist.science (the zh, fr and es
editions share its section numbering); "Veda news" is the aikraft.ru item on
Veda (ByteDance, HKU, USTC).  Where the pages leave a step open, the reading
taken is stated at the function that makes it (readings R1-R16 and R21-R28).

Every function works per attention head on numpy arrays and computes in
float64.  Inputs that are bf16 are widened exactly before they get here.

Parity pins: every function in this package is pinned by CPU tests to
something other than itself (brute force, closed forms, independent library
routines, invariants and hand-worked examples); none is "parity unpinned".
"""
from .tiling import tile_grid, slot_tokens, valid_slots, gather, scatter, HeadTiling
from .estimator import tripool, project, tile_scores
from .select import keep_count, select_topk
from .attention import sparse_attention, dense_attention, csr_to_block_mask
from .oracle_map import maxpool_map, maxpool_map_bruteforce
from .distill import kl_rows, distill_head
from .tiling_search import sparse_head_output, search_head
from .attention_bwd import sparse_attention_bwd

__all__ = [
    "tile_grid", "slot_tokens", "valid_slots", "gather", "scatter", "HeadTiling",
    "tripool", "project", "tile_scores", "keep_count", "select_topk",
    "sparse_attention", "dense_attention", "csr_to_block_mask",
    "maxpool_map", "maxpool_map_bruteforce", "kl_rows", "distill_head",
    "sparse_head_output", "search_head", "sparse_attention_bwd",
]
