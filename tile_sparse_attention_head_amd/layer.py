"""One tile-sparse attention layer on the GPU: buffers plus the call order.

``TileSparseAttention`` owns the device buffers one layer needs (allocated
once with torch; the library itself never allocates) and enqueues the
library's calls in the order of the method (Veda §2.1-§2.3).  ``forward``
runs the fused sequence:

  1. veda_tile_permute_pool  Q, K -> tile order, with their TripPool
                             descriptors; veda_tile_permute V -> tile-
                             transposed order
  2. veda_tile_score         per-head projection + tile scores
  3. veda_select_tiles       top-k key tiles per query tile -> CSR
  4. veda_sparse_attn_fwd_tokens   attention, O written in token order

(with ``score_select=True`` steps 2-3 are the projection alone and
veda_score_select, which never stores the score matrix: the same CSR).

``forward_unfused`` runs the same method one step per call (permute,
veda_tripool_score, select, veda_sparse_attn_fwd, inverse permute); both give
identical results.  ``maxpool_map`` runs veda_oracle_maxpool_map for a subset
of query tiles, ``distill_grad`` the estimator's distillation step
(veda_distill_grad) against that map, and ``backward`` the attention's
gradients (veda_sparse_attn_bwd).  All calls go on the current torch stream without
synchronising.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

from . import _lib as V


class TileSparseAttention:
    def __init__(self, T: int, H: int, W: int, head_dim: int, tile_size: int,
                 tile_shapes: Sequence[Tuple[int, int, int]], sparsity_pct: Optional[int] = None,
                 k_per_head: Optional[Sequence[int]] = None, d_e: Optional[int] = None,
                 device="cuda"):
        import torch
        self.torch = torch
        self.L = V.veda_layout_init(T, H, W, head_dim, tile_size, tile_shapes)
        L = self.L
        if k_per_head is None:
            if sparsity_pct is None:
                raise ValueError("give sparsity_pct or k_per_head")
            k_per_head = [V.veda_keep_count(L.n(h), sparsity_pct) for h in range(L.num_heads)]
        self.k_per_head = [int(v) for v in k_per_head]
        self.d_e = int(d_e or head_dim)
        self.nnz = V.csr_nnz(L, self.k_per_head)
        nt = V.tiles_numel(L)
        bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
        dev = torch.device(device)
        self.q_perm = torch.empty(nt, dtype=bf, device=dev)
        self.k_perm = torch.empty(nt, dtype=bf, device=dev)
        self.vt_perm = torch.empty(nt, dtype=bf, device=dev)
        self.o_perm = torch.empty(nt, dtype=bf, device=dev)
        self.lse = torch.empty(L.total_tiles * tile_size, dtype=f32, device=dev)
        self._map_ws = None   # veda_oracle_maxpool_map workspace, sized on first use
        self._distill_ws = None   # veda_distill_grad workspace, sized on first use
        self._bwd_ws = None       # veda_sparse_attn_bwd workspace, sized on first use
        # the attention forward's work counters (calls on one layer are ordered
        # on one stream)
        self._attn_ws = torch.empty(V.veda_sparse_attn_fwd_workspace(L), dtype=torch.uint8,
                                    device=dev)
        self.desc = torch.empty(2 * L.total_tiles * 3 * head_dim, dtype=f32, device=dev)
        self.phi = torch.empty(2 * L.total_tiles * self.d_e, dtype=f32, device=dev)
        self.scores = torch.empty(L.total_scores, dtype=f32, device=dev)
        self.row_ptr = torch.empty(L.total_tiles + 1, dtype=i32, device=dev)
        self.col_idx = torch.empty(max(1, self.nnz), dtype=i32, device=dev)

    # individual stages ---------------------------------------------------
    def permute_inputs(self, q, k, v, stream=None):
        V.veda_tile_permute(self.L, q, self.q_perm, V.VEDA_FWD, stream)
        V.veda_tile_permute(self.L, k, self.k_perm, V.VEDA_FWD, stream)
        V.veda_tile_permute(self.L, v, self.vt_perm, V.VEDA_FWD_T, stream)

    def score(self, w_q, w_k, b_q=None, b_k=None, stream=None):
        V.veda_tripool_score(self.L, self.q_perm, self.k_perm, w_q, w_k, self.desc, self.phi,
                             self.scores, b_q, b_k, stream)

    def select(self, stream=None):
        V.veda_select_tiles(self.L, self.scores, self.k_per_head, self.row_ptr, self.col_idx,
                            stream)

    def attend(self, sm_scale: float, with_lse: bool = True, stream=None):
        V.veda_sparse_attn_fwd(self.L, self.q_perm, self.k_perm, self.vt_perm, self.row_ptr,
                               self.col_idx, sm_scale, self.o_perm,
                               self.lse if with_lse else None, workspace=self._attn_ws,
                               stream=stream)

    def unpermute(self, out, stream=None):
        V.veda_tile_permute(self.L, self.o_perm, out, V.VEDA_INV, stream)

    # fused stages ------------------------------------------------------------
    def permute_pool_inputs(self, q, k, v, stream=None):
        """Q, K -> tile order with their TripPool descriptors (desc[0], desc[1]);
        V -> tile-transposed order."""
        n = self.L.total_tiles * 3 * self.L.head_dim
        V.veda_tile_permute_pool(self.L, q, self.q_perm, self.desc[:n], stream)
        V.veda_tile_permute_pool(self.L, k, self.k_perm, self.desc[n:2 * n], stream)
        V.veda_tile_permute(self.L, v, self.vt_perm, V.VEDA_FWD_T, stream)

    def score_from_desc(self, w_q, w_k, b_q=None, b_k=None, stream=None):
        V.veda_tile_score(self.L, self.desc, w_q, w_k, self.phi, self.scores, b_q, b_k, stream)

    def score_select_from_desc(self, w_q, w_k, b_q=None, b_k=None, stream=None):
        """Projection, then the scores and their top-k in one call
        (veda_score_select): the same CSR as score_from_desc + select, with
        ``scores`` left unwritten."""
        V.veda_tile_score(self.L, self.desc, w_q, w_k, self.phi, None, b_q, b_k, stream)
        V.veda_score_select(self.L, self.phi, self.d_e, self.k_per_head, self.row_ptr,
                            self.col_idx, stream)

    def attend_tokens(self, sm_scale: float, out, with_lse: bool = True, stream=None):
        V.veda_sparse_attn_fwd_tokens(self.L, self.q_perm, self.k_perm, self.vt_perm,
                                      self.row_ptr, self.col_idx, sm_scale, out,
                                      self.lse if with_lse else None, workspace=self._attn_ws,
                                      stream=stream)

    # whole layer -----------------------------------------------------------
    def forward(self, q, k, v, w_q, w_k, sm_scale: float, out=None, b_q=None, b_k=None,
                stream=None, score_select: bool = False):
        """q, k, v: bf16 [N][heads][d] (token order).  Returns O, same shape.
        score_select: scores and selection in one call (scores not stored)."""
        if out is None:
            out = self.torch.empty_like(q)
        self.permute_pool_inputs(q, k, v, stream)
        if score_select:
            self.score_select_from_desc(w_q, w_k, b_q, b_k, stream)
        else:
            self.score_from_desc(w_q, w_k, b_q, b_k, stream)
            self.select(stream)
        self.attend_tokens(sm_scale, out, True, stream)
        return out

    def forward_unfused(self, q, k, v, w_q, w_k, sm_scale: float, out=None, b_q=None, b_k=None,
                        stream=None):
        """forward, one method step per call (tile-order O, then the inverse
        permutation)."""
        if out is None:
            out = self.torch.empty_like(q)
        self.permute_inputs(q, k, v, stream)
        self.score(w_q, w_k, b_q, b_k, stream)
        self.select(stream)
        self.attend(sm_scale, True, stream)
        self.unpermute(out, stream)
        return out

    def backward(self, q, k, v, out, d_out, sm_scale: float, grads=None, stream=None,
                 reuse_tiles: bool = True):
        """dQ, dK, dV (token order) of the last ``forward`` (its inputs q, k,
        v and output ``out``, its lse and CSR still in this layer) for the
        output gradient ``d_out``.  With ``reuse_tiles`` the tile-order Q and
        K the forward gathered (still in this layer) are used instead of
        gathering q and k again; the results are the same."""
        torch = self.torch
        if grads is None:
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        need = V.veda_sparse_attn_bwd_workspace(self.L, self.nnz)
        if getattr(self, "_bwd_ws", None) is None or self._bwd_ws.numel() < need:
            self._bwd_ws = torch.empty(max(16, need), dtype=torch.uint8, device=q.device)
        if reuse_tiles:
            V.veda_sparse_attn_bwd_tiles(self.L, self.q_perm, self.k_perm, v, out, d_out,
                                         self.lse, self.row_ptr, self.col_idx, self.nnz,
                                         sm_scale, self._bwd_ws, *grads, stream=stream)
        else:
            V.veda_sparse_attn_bwd(self.L, q, k, v, out, d_out, self.lse, self.row_ptr,
                                   self.col_idx, self.nnz, sm_scale, self._bwd_ws, *grads,
                                   stream=stream)
        return grads

    def maxpool_map(self, q_tiles, sm_scale: float, lse=None, out_map=None, stream=None):
        """Max-pooled map of the query tiles ``q_tiles`` (int32 global tile
        indices) over the tile-ordered Q, K already in this layer's buffers."""
        torch = self.torch
        n_sub = int(q_tiles.numel())
        if lse is None:
            lse = torch.empty(max(1, n_sub * self.L.tile_size), dtype=torch.float32,
                              device=self.q_perm.device)
        if out_map is None:
            out_map = torch.empty(max(1, n_sub * self.L.max_tiles), dtype=torch.float32,
                                  device=self.q_perm.device)
        need = V.veda_oracle_maxpool_map_workspace(self.L, n_sub)
        if self._map_ws is None or self._map_ws.numel() < need:
            # kept across calls; the pass-1 row maxima live here
            self._map_ws = torch.empty(max(16, need), dtype=torch.uint8, device=self.q_perm.device)
        V.veda_oracle_maxpool_map(self.L, self.q_perm, self.k_perm, sm_scale, q_tiles,
                                  self._map_ws, lse, out_map, stream)
        return lse, out_map

    def distill_grad(self, q_tiles, out_map, loss=None, grads=None, with_bias=True, stream=None):
        """Row-wise KL distillation loss of the scores this layer last computed
        against the max-pooled map ``out_map`` of ``q_tiles``, and the
        gradients of the projections (Veda §2.1 optimisation).  Returns
        (loss [1], (grad_w_q, grad_w_k, grad_b_q, grad_b_k))."""
        torch = self.torch
        L, dev = self.L, self.q_perm.device
        n_sub = int(q_tiles.numel())
        H, de, d3 = L.num_heads, self.d_e, 3 * L.head_dim
        if loss is None:
            loss = torch.empty(1, dtype=torch.float32, device=dev)
        if grads is None:
            grads = (torch.empty(H, de, d3, dtype=torch.float32, device=dev),
                     torch.empty(H, de, d3, dtype=torch.float32, device=dev),
                     torch.empty(H, de, dtype=torch.float32, device=dev) if with_bias else None,
                     torch.empty(H, de, dtype=torch.float32, device=dev) if with_bias else None)
        need = V.veda_distill_grad_workspace(L, n_sub, de)
        if getattr(self, "_distill_ws", None) is None or self._distill_ws.numel() < need:
            self._distill_ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
        V.veda_distill_grad(L, self.scores, out_map, q_tiles, self.desc, self.phi, de,
                            self._distill_ws, loss, *grads, stream=stream)
        return loss, grads
