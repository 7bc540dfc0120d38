"""Head-aware tiling search (Veda §2.2: configuration search, offline
selection): for every head, the candidate tile shape whose sparse attention
output is closest to full attention on calibration inputs.

Host orchestration of the library's calls; every step on the data runs in
the HIP kernels:

  1. full attention of the calibration layer: the fused layer with every key
     tile kept (0 % sparsity), which is exact dense attention over the real
     tokens whatever the tiling;
  2. for each candidate shape (all heads at once): the fused layer at the
     requested sparsity, then veda_head_sq_error against step 1;
  3. veda_head_choose: per head, the candidate with the smallest squared
     error (equal errors prefer the earlier candidate).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

from . import _lib as V
from .layer import TileSparseAttention

# the four factorisations of a 128-slot hardware tile the pages search over
SHAPES_128 = [(1, 8, 16), (2, 8, 8), (4, 4, 8), (8, 4, 4)]


def search_tile_shapes(T: int, H: int, W: int, head_dim: int, tile_size: int, q, k, v, w_q, w_k,
                       sm_scale: float, sparsity_pct: int,
                       candidates: Sequence[Tuple[int, int, int]] = SHAPES_128,
                       b_q=None, b_k=None, stream=None):
    """q, k, v: bf16 [N][heads][d] token order; w_q, w_k: f32 [heads][d_e][3d].

    Returns (chosen shape per head, errors f64 [len(candidates)][heads],
    ref f64 [heads] = squared norm of full attention per head), errors and ref
    as device tensors."""
    import torch
    heads = int(q.shape[1])
    dev = q.device
    full_layer = TileSparseAttention(T, H, W, head_dim, tile_size, [tuple(candidates[0])] * heads,
                                     sparsity_pct=0, device=dev)
    full = full_layer.forward(q, k, v, w_q, w_k, sm_scale, b_q=b_q, b_k=b_k, stream=stream)
    ws = torch.empty(max(8, V.veda_head_sq_error_workspace(full_layer.L)), dtype=torch.uint8,
                     device=dev)
    del full_layer
    errs = torch.empty(len(candidates), heads, dtype=torch.float64, device=dev)
    ref = torch.empty(heads, dtype=torch.float64, device=dev)
    out = torch.empty_like(q)
    for c, shape in enumerate(candidates):
        ly = TileSparseAttention(T, H, W, head_dim, tile_size, [tuple(shape)] * heads,
                                 sparsity_pct=sparsity_pct, device=dev)
        ly.forward(q, k, v, w_q, w_k, sm_scale, out=out, b_q=b_q, b_k=b_k, stream=stream)
        V.veda_head_sq_error(ly.L, full, out, errs[c], ws, ref=ref if c == 0 else None,
                             stream=stream)
        del ly
    choice = torch.empty(heads, dtype=torch.int32, device=dev)
    V.veda_head_choose(errs, choice, stream=stream)
    # the chosen shapes are host parameters of the layers built from them
    chosen: List[Tuple[int, int, int]] = [tuple(candidates[int(c)]) for c in choice.cpu()]
    return chosen, errs, ref
