"""Tile selection at a fixed sparsity, emitted as CSR.

Veda summary (lay part and §5) and Veda news: at 95 % sparsity each query
tile keeps about 5 % of the key/value tiles, chosen by the estimator's
tile-level scores; the tile-skipping kernel then reads only the kept tiles.

Readings:
  R10 sparsity counts key tiles per query-tile row: a head with n tiles keeps
      k = max(1, ceil(n * (100 - s) / 100)) of them, in integer arithmetic.
  R11 the kept tiles are the k largest scores; equal scores prefer the lower
      tile index; -0.0 equals +0.0; NaN ranks below every number (NaNs among
      themselves by index).
  R12 each CSR row lists its kept tile indices in ascending order.
  R13 no tile is forced in (pure top-k).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def keep_count(n_tiles: int, sparsity_pct: int) -> int:
    """Key tiles kept per query tile at ``sparsity_pct`` percent sparsity (R10)."""
    n, s = int(n_tiles), int(sparsity_pct)
    if not (0 <= s <= 100) or n < 1:
        raise ValueError("bad n_tiles / sparsity")
    return max(1, -(-(n * (100 - s)) // 100))


def select_topk(scores: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise top-k of one head's [n][n] score matrix as CSR (R11, R12).

    Returns (row_ptr [n+1], col_idx [n*k]) with head-local tile indices.
    """
    s = np.asarray(scores, dtype=np.float64)
    n_rows, n_cols = s.shape
    if not 1 <= k <= n_cols:
        raise ValueError("k out of range")
    row_ptr = np.arange(n_rows + 1, dtype=np.int64) * k
    col_idx = np.empty(n_rows * k, dtype=np.int64)
    idx = np.arange(n_cols)
    for i in range(n_rows):
        row = s[i]
        is_nan = np.isnan(row)
        neg = np.where(is_nan, 0.0, -row)
        # primary: numbers before NaN; then larger score first; then lower index
        order = np.lexsort((idx, neg, is_nan))
        col_idx[i * k:(i + 1) * k] = np.sort(order[:k])
    return row_ptr, col_idx
