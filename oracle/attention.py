"""Softmax attention restricted to the kept tiles, and dense attention.

Veda §2.3 (hardware-efficient implementation): the tile-skipping kernel
computes attention of each query tile against only its kept, non-contiguous
key/value tiles; everything it skips contributes nothing.  Veda §1 states the
dense O(N^2) self-attention this replaces.  So for query row r of tile i

    l_rc  = sm_scale * q_r . k_c       for the valid key slots c of kept tiles
    lse_r = log sum_c exp(l_rc)
    o_r   = sum_c exp(l_rc - lse_r) v_c

Readings:
  R9  sm_scale is an explicit argument (the pages give none).
  R14 padding key slots are excluded from the softmax (so that keeping every
      tile reproduces dense attention over the real tokens).
  R15 outputs of padding query slots are unspecified: returned as NaN here.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np


def _softmax_rows(logits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    ssum = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(ssum))[:, 0]
    return e / ssum, lse


def sparse_attention(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, valid: np.ndarray,
                     S: int, row_ptr: np.ndarray, col_idx: np.ndarray, sm_scale: float,
                     q_tiles: Optional[Iterable[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Block-sparse attention of one head in tile order.

    ``qp, kp, vp``: [n*S][d] tile-ordered (padding rows are zero);
    ``row_ptr, col_idx``: head-local CSR of kept key tiles per query tile;
    ``q_tiles``: optional subset of query tiles to compute (others stay NaN).
    Returns (o [n*S][d], lse [n*S]) with NaN at padding and uncomputed rows.
    """
    q = np.asarray(qp, np.float64)
    k = np.asarray(kp, np.float64)
    v = np.asarray(vp, np.float64)
    n = q.shape[0] // S
    o = np.full(q.shape[:1] + v.shape[1:], np.nan)
    lse = np.full(q.shape[0], np.nan)
    tiles = range(n) if q_tiles is None else q_tiles
    for i in tiles:
        kept = col_idx[row_ptr[i]:row_ptr[i + 1]]
        key_slots = np.concatenate([np.arange(j * S, (j + 1) * S) for j in kept])
        key_slots = key_slots[valid[key_slots]]
        q_slots = np.arange(i * S, (i + 1) * S)
        q_slots = q_slots[valid[q_slots]]
        logits = sm_scale * (q[q_slots] @ k[key_slots].T)
        p, l = _softmax_rows(logits)
        o[q_slots] = p @ v[key_slots]
        lse[q_slots] = l
    return o, lse


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Dense softmax attention of one head in token order, no tiling
    (Veda §1: every token attends to every token).  Returns (o, lse)."""
    logits = sm_scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    p, lse = _softmax_rows(logits)
    return p @ np.asarray(v, np.float64), lse


def csr_to_block_mask(row_ptr: np.ndarray, col_idx: np.ndarray, valid: np.ndarray,
                      S: int) -> np.ndarray:
    """Boolean [n*S][n*S] mask (query slot, key slot) allowed by the CSR:
    the key slot is valid and its tile is kept by the query slot's tile."""
    n = valid.size // S
    tile_keep = np.zeros((n, n), dtype=bool)
    for i in range(n):
        tile_keep[i, col_idx[row_ptr[i]:row_ptr[i + 1]]] = True
    mask = np.repeat(np.repeat(tile_keep, S, axis=0), S, axis=1)
    return mask & valid[None, :]
