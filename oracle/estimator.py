"""Distilled tile-score estimator: TripPool descriptor, per-head projection,
tile-pair score.

Veda §2.1 (distilled tile scoring): a light estimator predicts tile-level
attention scores; each tile is described by TripPool, the concatenation of the
mean, maximum and minimum statistics of its tokens, and each attention head
has its own MLP projection of that descriptor.

Readings (the pages leave these open):
  R5  the statistics are taken per channel over the tile's real (non-padding)
      tokens, concatenated in the order mean, max, min  -> 3d values.
  R6  the projection is one linear map 3d -> d_e with an optional bias and no
      activation.
  R7  the query-side and key-side descriptors each go through a projection of
      their own head (the two weight sets may be equal).
  R8  the score of query tile i against key tile j is the plain inner product
      of the two projected descriptors (no temperature: top-k is invariant to
      any positive scale).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def tripool(x_perm: np.ndarray, valid: np.ndarray, S: int) -> np.ndarray:
    """TripPool descriptor of every tile of one head (R5).

    ``x_perm`` is [n*S][d] in tile order, ``valid`` the slot mask.  Returns
    [n][3d] = [mean | max | min] over the tile's valid slots, per channel.
    """
    x = np.asarray(x_perm, dtype=np.float64)
    n = x.shape[0] // S
    d = x.shape[1]
    out = np.empty((n, 3 * d), dtype=np.float64)
    for j in range(n):
        rows = x[j * S:(j + 1) * S][valid[j * S:(j + 1) * S]]
        out[j, 0:d] = rows.sum(axis=0) / rows.shape[0]
        out[j, d:2 * d] = rows.max(axis=0)
        out[j, 2 * d:3 * d] = rows.min(axis=0)
    return out


def project(desc: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-head projection phi = W desc (+ b)  (R6).  ``w`` is [d_e][3d]."""
    phi = np.asarray(desc, np.float64) @ np.asarray(w, np.float64).T
    if b is not None:
        phi = phi + np.asarray(b, np.float64)[None, :]
    return phi


def tile_scores(phi_q: np.ndarray, phi_k: np.ndarray) -> np.ndarray:
    """Tile-pair scores of one head: score[i][j] = <phi_q[i], phi_k[j]>  (R8)."""
    return np.asarray(phi_q, np.float64) @ np.asarray(phi_k, np.float64).T
