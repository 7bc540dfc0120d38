"""Head-aware tiling search: per head, the tile shape whose sparse attention is
closest to full attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Veda §2.2 (head-aware tiling; configuration search, offline selection): for
every layer and head the tile shape pi = (pt, ph, pw) factorising the hardware
tile is chosen offline, as the one that minimises the approximation error
between the full-attention output and the sparse-attention output on a
calibration set.

Readings (the pages leave these open):
  R25 the sparse output is the method as it runs: TripPool + projection +
      score, top-k at the given sparsity, tile-skipping attention, back to
      token order;
  R26 the error of a head is the squared Frobenius norm of the difference of
      its two outputs over the real tokens; the relative error divides it by
      the squared norm of the full-attention output;
  R27 the candidates are the shapes given (the pages' four for S = 128);
      equal errors prefer the earlier candidate.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .attention import dense_attention, sparse_attention
from .estimator import project, tile_scores, tripool
from .select import keep_count, select_topk
from .tiling import HeadTiling, gather, scatter


def sparse_head_output(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: int, H: int, W: int,
                       shape: Tuple[int, int, int], w_q: np.ndarray, w_k: np.ndarray,
                       b_q: Optional[np.ndarray], b_k: Optional[np.ndarray], sm_scale: float,
                       sparsity_pct: int) -> np.ndarray:
    """One head's sparse-attention output in token order with tile shape
    ``shape`` (R25): ``q, k, v`` [N][d] token order, fp64."""
    ht = HeadTiling(T, H, W, shape)
    qp, kp, vp = (gather(a, T, H, W, shape) for a in (q, k, v))
    s = tile_scores(project(tripool(qp, ht.valid, ht.S), w_q, b_q),
                    project(tripool(kp, ht.valid, ht.S), w_k, b_k))
    rp, ci = select_topk(s, keep_count(ht.n, sparsity_pct))
    o, _ = sparse_attention(qp, kp, vp, ht.valid, ht.S, rp, ci, sm_scale)
    return scatter(np.nan_to_num(o), T, H, W, shape)


def search_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: int, H: int, W: int,
                candidates: Sequence[Tuple[int, int, int]], w_q: np.ndarray, w_k: np.ndarray,
                b_q: Optional[np.ndarray], b_k: Optional[np.ndarray], sm_scale: float,
                sparsity_pct: int):
    """Squared error of every candidate shape for one head (R26) and the
    chosen one (R27).  Returns (errors [len(candidates)], ref = ||O_full||^2,
    index of the chosen candidate)."""
    full, _ = dense_attention(q, k, v, sm_scale)
    errs = np.array([((full - sparse_head_output(q, k, v, T, H, W, c, w_q, w_k, b_q, b_k,
                                                 sm_scale, sparsity_pct)) ** 2).sum()
                     for c in candidates])
    return errs, float((full ** 2).sum()), int(np.argmin(errs))
