"""Distillation objective of the tile-score estimator and its gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Veda §2.1 (distilled tile scoring, optimisation): the estimator is trained
with a row-wise KL-divergence objective that aligns the distribution of its
predicted tile scores with the full-attention reference, and a stop-gradient
on the backbone features that feed the estimator, so only the estimator's own
parameters learn.

Readings (the pages leave these open):
  R21 the predicted distribution of query tile i is the softmax over the
      head's key tiles j of the estimator score S[i][j] (no temperature);
  R22 the reference distribution is the max-pooled map row M[i][:] (Veda
      §2.1 target construction; ``maxpool_map``) divided by its sum;
  R23 the divergence is KL(reference || predicted) = sum_j t_j log(t_j/p_j),
      with t_j log t_j = 0 for t_j = 0, averaged over the subset's query-tile
      rows of every head (R = number of rows);
  R24 stop-gradient on the features means the TripPool descriptors are
      constants: gradients flow to the projection weights and biases only;
      the query-side and key-side projections get gradients of their own
      (equal weight sets are one parameter whose gradient is the sum).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .estimator import project, tile_scores


def kl_rows(scores_rows: np.ndarray, map_rows: np.ndarray) -> np.ndarray:
    """KL(t || p) of every row (R21-R23): ``scores_rows`` [R][n] estimator
    scores, ``map_rows`` [R][n] max-pooled map, each row with a positive sum."""
    s = np.asarray(scores_rows, np.float64)
    m = np.asarray(map_rows, np.float64)
    z = s - s.max(axis=1, keepdims=True)
    log_p = z - np.log(np.exp(z).sum(axis=1, keepdims=True))
    t = m / m.sum(axis=1, keepdims=True)
    safe_t = np.where(t > 0, t, 1.0)
    return np.where(t > 0, t * (np.log(safe_t) - log_p), 0.0).sum(axis=1)


def distill_head(desc_q: np.ndarray, desc_k: np.ndarray, w_q: np.ndarray, w_k: np.ndarray,
                 b_q: Optional[np.ndarray], b_k: Optional[np.ndarray], rows: Sequence[int],
                 map_rows: np.ndarray, n_rows_total: int):
    """One head's share of the objective and of its gradients.

    ``desc_q``/``desc_k`` [n][3d] TripPool descriptors (constants, R24);
    ``w_*`` [d_e][3d], ``b_*`` [d_e] or None; ``rows`` the head-local query
    tiles of the subset (repeats allowed), ``map_rows`` [len(rows)][n] their
    max-pooled map rows; ``n_rows_total`` = R over all heads.

    Returns (loss share, dW_q, dW_k, db_q, db_k): the loss share is
    sum over this head's rows of KL / R.
    """
    rows = np.asarray(rows, np.int64)
    R = float(n_rows_total)
    phi_q = project(desc_q, w_q, b_q)              # forward (Veda §2.1 estimator)
    phi_k = project(desc_k, w_k, b_k)
    s = tile_scores(phi_q, phi_k)
    loss = kl_rows(s[rows], map_rows).sum() / R
    # dL/dS[rows[r]][j] = (p - t) / R  (softmax-KL gradient, one row per subset entry)
    z = s[rows] - s[rows].max(axis=1, keepdims=True)
    p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    t = np.asarray(map_rows, np.float64) / np.asarray(map_rows, np.float64).sum(axis=1, keepdims=True)
    g = (p - t) / R                                 # [len(rows)][n]
    # S = phi_q phi_k^T: dphi_q[i] = sum over entries r with rows[r] = i of g[r] phi_k
    dphi_q = np.zeros_like(phi_q)
    np.add.at(dphi_q, rows, g @ phi_k)
    dphi_k = g.T @ phi_q[rows]
    # phi = desc W^T + b
    dw_q = dphi_q.T @ np.asarray(desc_q, np.float64)
    dw_k = dphi_k.T @ np.asarray(desc_k, np.float64)
    return loss, dw_q, dw_k, dphi_q.sum(axis=0), dphi_k.sum(axis=0)
